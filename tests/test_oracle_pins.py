"""Pins for the CPU oracle: each check ties an oracle function to something other
than itself -- exact rational arithmetic, brute force over tiny inputs, closed
forms, or an independent library routine.  ``test_planted_mistakes`` then
plants plausible mistakes in the oracle (on the CPU) and requires that some
check catches every one of them.

Page references: MemLong section 2.3.2 (cosine top-k over chunk embeddings;
memory of K-V plus index-aligned embeddings), Figure 3 (retrieved chunks fully
visible, local context causal); InfLLM "method" (window + block memory units
with representative tokens); Landmark Attention "proposed method" (one
landmark per fixed-length block, query-landmark similarity decides retrieval);
MoNIM section 2.1 (kNN lookup over a key-value store: the token-level special
case used below).
"""
from __future__ import annotations

import itertools
import math
import random
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.brs_oracle as O

# ---------------------------------------------------------------------------
# independent exact helpers (Fraction arithmetic)


def rne_fraction(x: Fraction, p: int, emin: int = -126) -> Fraction:
    """Exact round-to-nearest-even of a rational to p significand bits."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    unit = Fraction(2) ** (e - p + 1)
    n = round(x / unit)  # Fraction.__round__ rounds half to even
    return n * unit


def exact(v) -> Fraction:
    return Fraction(float(v))


def bf16_values(rng, shape) -> np.ndarray:
    """float64 array of exact bfloat16 values (independent of the oracle's rounding)."""
    t = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# checks (reach the oracle through the module so mistakes can be planted)


def check_round_f32():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 38, 4000),
                        [1e-45, 3e-39, -2.5e-40, 3.4028235e38, 3.5e38, 1 + 2 ** -24, 1 + 3 * 2 ** -24]])
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).astype(np.float64)
    got = O.round_to_dtype(x, "f32")
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def check_round_bf16():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.4028235e38, 1e-39], dtype=np.float32)
    x32 = np.concatenate([x32, ties])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_dtype(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]
    # float64 inputs: compare with exact rational rounding (no double rounding)
    x64 = rng.standard_normal(300) * 3
    got = O.round_to_dtype(x64, "bf16")
    for a, b in zip(x64, got):
        assert Fraction(float(b)) == rne_fraction(Fraction(float(a)), 8)


def check_eligible_bruteforce():
    for N in range(1, 70):
        for B in (1, 2, 3, 5, 8, 16):
            for S in (0, 1, 3, 7, 16, 40):
                for W in (0, 1, 4, 9, 16, 33, 80):
                    nb = N // B
                    union = set(range(min(S, N))) | set(range(max(N - W, 0), N))
                    want = [b for b in range(nb) if any(t not in union for t in range(b * B, (b + 1) * B))]
                    lo, hi = O.eligible_range(N, B, S, W)
                    assert list(range(lo, hi)) == want, (N, B, S, W, lo, hi, want)


def check_eligible_workloads():
    # closed form evaluated by hand for the five workloads
    assert O.eligible_range(4096, 64, 4, 256) == (0, 60)
    assert O.eligible_range(32768, 50, 0, 512) == (0, 646)
    assert O.eligible_range(131072, 128, 128, 4096) == (1, 992)
    assert O.eligible_range(82432, 512, 0, 512) == (0, 160)
    assert O.eligible_range(1048576, 64, 0, 0) == (0, 16384)


def check_mean_exact():
    rng = np.random.default_rng(3)
    for dtype, p in (("bf16", 8), ("f32", 24)):
        for B in (1, 3, 64):
            K = bf16_values(rng, (B * 4 + B // 2, 5)) if dtype == "bf16" else \
                rng.standard_normal((B * 4 + B // 2, 5)).astype(np.float32).astype(np.float64)
            got = O.reps_mean(K, B, dtype)
            assert got.shape == (4, 1, 5)
            for b in range(4):
                for i in range(5):
                    s = sum(exact(K[t, i]) for t in range(b * B, (b + 1) * B))
                    assert exact(got[b, 0, i]) == rne_fraction(s / B, p)
    # a block of identical keys has that key as its mean
    K = np.repeat(bf16_values(rng, (1, 8)), 64, axis=0)
    assert np.array_equal(O.reps_mean(K, 64, "bf16")[0, 0], K[0])


def check_topnorm_bruteforce():
    rng = random.Random(4)
    for trial in range(60):
        B, R, d = rng.randint(1, 7), rng.randint(1, 4), rng.randint(1, 4)
        R = min(R, B)
        vals = [[rng.choice([-2, -1, 0, 1, 2, 0.5, 3]) for _ in range(d)] for _ in range(2 * B)]
        K = np.array(vals, dtype=np.float64)
        got = O.reps_topnorm(K, B, R)
        for b in range(2):
            toks = list(range(b * B, (b + 1) * B))
            norms = {t: sum(Fraction(x) ** 2 for x in vals[t]) for t in toks}
            # brute force: the ordered R-tuple that no other ordering beats
            best = max(itertools.permutations(toks, R),
                       key=lambda perm: [(norms[t], -t) for t in perm])
            assert np.array_equal(got[b], K[list(best)]), (trial, b)
    # one key scaled up becomes the first representative
    K = np.array([[1.0, 0.0], [0.0, 1.0], [10.0, 0.0], [0.5, 0.5]])
    assert np.array_equal(O.reps_topnorm(K, 4, 1)[0, 0], [10.0, 0.0])
    # equal norms: lower token first
    K = np.array([[0.0, 2.0], [2.0, 0.0], [-2.0, 0.0], [1.0, 1.0]])
    assert np.array_equal(O.reps_topnorm(K, 4, 3)[0], K[[0, 1, 2]])


def check_dot_exact_mips():
    """B = 1, R = 1: scores are exact maximum-inner-product values over the keys
    (the kNN key-value lookup of MoNIM section 2.1), rounded once to float32."""
    rng = np.random.default_rng(5)
    for d in (4, 64, 128):
        q = bf16_values(rng, (d,))
        keys = bf16_values(rng, (50, d))
        got = O.scores_dot_max(q, keys[:, None, :])
        for b in range(50):
            s = sum(exact(q[i]) * exact(keys[b, i]) for i in range(d))
            assert Fraction(float(got[b])) == rne_fraction(s, 24), (d, b)
    # hand example and max over representatives
    q = np.array([1.0, 2.0])
    reps = np.array([[[3.0, 4.0]], [[-1.0, 0.0]]])
    assert O.scores_dot_max(q, reps).tolist() == [11.0, -1.0]
    reps2 = np.array([[[1.0, 0.0], [0.0, 5.0], [2.0, 2.0]]])
    assert O.scores_dot_max(q, reps2).tolist() == [10.0]
    # R copies of one representative score like that representative
    r = bf16_values(rng, (7, 1, 128))
    q = bf16_values(rng, (128,))
    assert np.array_equal(O.scores_dot_max(q, np.repeat(r, 4, axis=1)), O.scores_dot_max(q, r))


def check_group_max():
    """Group scores (one selection per kv head): brute force over every
    (head, representative) pair on small integer vectors, whose dots are
    exact in float32; a group of one head is the per-head score; the head
    order and a repeated head change nothing; a block planted for one head
    of the group wins the group's selection."""
    rng = np.random.default_rng(18)
    for trial in range(20):
        G, nb, R, d = int(rng.integers(1, 5)), int(rng.integers(1, 7)), int(rng.integers(1, 4)), 6
        Qg = rng.integers(-4, 5, size=(G, d)).astype(np.float64)
        reps = rng.integers(-4, 5, size=(nb, R, d)).astype(np.float64)
        want = [max(sum(int(Qg[h, i]) * int(reps[b, r, i]) for i in range(d)) for h in range(G) for r in range(R))
                for b in range(nb)]
        assert O.scores_group_max(Qg, reps).tolist() == [float(v) for v in want], trial
        perm = rng.permutation(G)
        assert np.array_equal(O.scores_group_max(Qg[perm], reps), O.scores_group_max(Qg, reps))
        assert np.array_equal(O.scores_group_max(np.concatenate([Qg, Qg[:1]]), reps), O.scores_group_max(Qg, reps))
    q = bf16_values(rng, (1, 64))
    reps = bf16_values(rng, (30, 2, 64))
    assert np.array_equal(O.scores_group_max(q, reps), O.scores_dot_max(q[0], reps))
    # planted: block 17 carries 0.8 q of head 2 of 4
    Qg = bf16_values(rng, (4, 64))
    reps = bf16_values(rng, (40, 1, 64))
    reps[17, 0] = 0.8 * Qg[2] + 0.1 * reps[17, 0]
    idx, _ = O.select_topk(O.scores_group_max(Qg, reps), 0, 40, 1)
    assert idx.tolist() == [17]
    # one step with group selection: every head of a kv head attends the same blocks
    Hq, Hkv, N, B, dd = 4, 2, 160, 16, 8
    qs = rng.standard_normal((1, Hq, 1, dd))
    K = rng.standard_normal((1, Hkv, N, dd))
    V = rng.standard_normal((1, Hkv, N, dd))
    rp = np.stack([np.stack([O.reps_mean(K[0, g], B, "f32") for g in range(Hkv)])])
    res = O.step(qs, K, V, rp, block=B, k=3, sinks=0, window=16, mode="mean", select="group")
    for g in range(Hkv):
        sg = O.scores_group_max(qs[0, 2 * g:2 * g + 2, -1], rp[0, g, 0:9])
        assert np.array_equal(res["scores"][(0, g)][0:9], sg)
        for h in (2 * g, 2 * g + 1):
            T = O.attended_mask(N, B, 0, 16, res["idx"][(0, g)])
            assert np.array_equal(res["out"][(0, h)], O.attention(qs[0, h], K[0, g], V[0, g], T, 1 / math.sqrt(dd)))
    one = O.step(qs[:, :2], K[:, :2], V[:, :2], rp[:, :2], block=B, k=3, sinks=0, window=16, mode="mean")
    same = O.step(qs[:, :2], K[:, :2], V[:, :2], rp[:, :2], block=B, k=3, sinks=0, window=16, mode="mean",
                  select="group")
    for h in range(2):
        assert np.array_equal(one["idx"][(0, h)], same["idx"][(0, h)])


def check_cosine():
    from scipy.spatial.distance import cosine as scipy_cosine_distance

    rng = np.random.default_rng(6)
    rq = bf16_values(rng, (768,))
    E = bf16_values(rng, (40, 768))
    got = O.scores_cosine(rq, E)
    want = np.array([1.0 - scipy_cosine_distance(rq, e) for e in E])
    assert np.max(np.abs(got - want)) < 2e-7
    # cos(x, x) = 1, cos(x, -x) = -1, zero vector scores 0
    E2 = np.stack([rq, -rq, np.zeros(768), 2.0 * rq])
    assert O.scores_cosine(rq, E2).tolist() == [1.0, -1.0, 0.0, 1.0]
    assert O.scores_cosine(np.zeros(768), E).tolist() == [0.0] * 40
    # scale invariance (power-of-two scales are exact)
    assert np.array_equal(O.scores_cosine(4.0 * rq, 0.5 * E), got)
    # unit-norm inputs: a plain dot product
    u = rq / np.linalg.norm(rq)
    V = E / np.linalg.norm(E, axis=1, keepdims=True)
    assert np.max(np.abs(O.scores_cosine(u, V) - (V @ u))) < 1e-7


def _f32_from_decimal(c):
    """The float32 nearest to the Decimal c, ties to even, decided with Decimal midpoints."""
    f0 = np.float32(float(c))
    cands = [np.nextafter(f0, np.float32(-np.inf)), f0, np.nextafter(f0, np.float32(np.inf))]
    best = cands[0]
    for c0, c1 in zip(cands, cands[1:]):
        mid = (Decimal(float(c0)) + Decimal(float(c1))) / 2
        if c > mid:
            best = c1
        elif c == mid:
            best = c0 if (int(np.float32(c0).view(np.uint32)) & 1) == 0 else c1
            break
        else:
            break
    return float(best)


def cosine_decimal(rq, e):
    """Cosine of two float64 vectors in 400-digit decimal arithmetic (their
    products and sums exact at this precision), rounded once to float32."""
    with localcontext() as ctx:
        ctx.prec = 400
        xs = [Decimal(float(v)) for v in rq]
        ys = [Decimal(float(v)) for v in e]
        dot = sum(x * y for x, y in zip(xs, ys))
        qq = sum(x * x for x in xs)
        ee = sum(y * y for y in ys)
        if qq == 0 or ee == 0:
            return 0.0
        return _f32_from_decimal(dot / (qq.sqrt() * ee.sqrt()))


def near_tie_cosine_cases(n_cases: int, seed: int):
    """Vectors whose cosine lies within 2**-53 (relative) of a float32
    rounding midpoint, so that float64 evaluations of the formula fall on
    either side of it.  rq is 768 ones and e holds integers below 2**24 with
    sum S1 and square sum S2, so cos = S1 / sqrt(768 S2) exactly; S2 is the
    integer (of the parity of S1) nearest to S1**2 / (768 m**2) for a float32
    midpoint m, with S2 about 2**52."""
    rng = random.Random(seed)
    n = 768
    out = []
    for _ in range(n_cases):
        f = np.float32(rng.uniform(0.05, 0.95))
        m = (Fraction(float(f)) + Fraction(float(np.nextafter(f, np.float32(2.0))))) / 2
        S1 = int(m * math.isqrt(n << 52)) + rng.randint(-999, 999)
        target = Fraction(S1 * S1) / (n * m * m)
        S2 = round(target)
        if (S2 - S1) % 2:
            S2 += 1 if S2 < target else -1
        v, r = divmod(S1, n)
        e = [v + 1] * r + [v] * (n - r)
        gap = S2 - sum(x * x for x in e)
        assert gap >= 0 and gap % 2 == 0
        i = 0
        while gap:  # move pairs of equal entries apart: +d and -d add 2 d**2
            assert e[i] == e[i + 1]
            d = max(1, min(math.isqrt(gap // 2), (1 << 24) - 1 - abs(e[i])))
            e[i] += d
            e[i + 1] -= d
            gap -= 2 * d * d
            i += 2
        assert sum(e) == S1 and sum(x * x for x in e) == S2 and max(abs(x) for x in e) < 1 << 24
        out.append((np.ones(n), np.array(e, dtype=np.float64)))
    return out


def check_cosine_exact_rounding():
    """The cosine is the exact value rounded once to float32: equal, bit for
    bit, to a 400-digit decimal evaluation rounded to the nearest float32 --
    on random bfloat16 vectors and on vectors whose cosine sits within 2**-53
    of a float32 rounding midpoint, where float64 formulas disagree."""
    rng = np.random.default_rng(16)
    rq = bf16_values(rng, (768,))
    E = bf16_values(rng, (12, 768))
    got = O.scores_cosine(rq, E)
    for b in range(E.shape[0]):
        assert float(got[b]) == cosine_decimal(rq, E[b]), b
    ties = near_tie_cosine_cases(24, 17)
    wrong_a = wrong_b = 0
    for (q, e) in ties:
        want = cosine_decimal(q, e)
        assert float(O.scores_cosine(q, e[None])[0]) == want
        qq, ee, dot = float(q @ q), float(e @ e), float(q @ e)
        wrong_a += float(np.float32(dot / (math.sqrt(qq) * math.sqrt(ee)))) != want
        wrong_b += float(np.float32(dot / math.sqrt(qq * ee))) != want
    # the cases separate the exact value from both float64 formulas
    assert wrong_a > 0 and wrong_b > 0, (wrong_a, wrong_b)


def _key(s, b):
    return (1, 0.0, b) if math.isnan(s) else (0, -s, b)


def check_topk_bruteforce():
    rng = random.Random(7)
    for trial in range(300):
        n = rng.randint(1, 8)
        s = np.array([rng.choice([0.5, 1.0, 1.0, -2.0, 3.0, float("nan"), 7.25]) for _ in range(n)],
                     dtype=np.float32)
        lo = rng.randint(0, n)
        hi = rng.randint(lo, n)
        k = rng.randint(1, n + 2)
        idx, vals = O.select_topk(s, lo, hi, k)
        m = min(k, hi - lo)
        # exhaustive: the one m-subset whose every member beats every non-member
        cands = range(lo, hi)
        winners = [c for c in itertools.combinations(cands, m)
                   if all(_key(s[a], a) < _key(s[z], z) for a in c for z in cands if z not in c)]
        assert len(winners) == 1
        want = sorted(winners[0], key=lambda b: _key(s[b], b))
        assert idx[:m].tolist() == list(want), (trial, s, lo, hi, k, idx)
        assert idx[m:].tolist() == [-1] * (k - m)
        assert np.array_equal(vals[:m], s[list(want)], equal_nan=True)
        assert np.all(np.isneginf(vals[m:]))


def check_topk_ties_and_nan():
    s = np.array([1.0, 5.0, 5.0, np.nan, 5.0, 2.0], dtype=np.float32)
    idx, _ = O.select_topk(s, 0, 6, 6)
    assert idx.tolist() == [1, 2, 4, 5, 0, 3]
    idx, _ = O.select_topk(s, 2, 6, 2)
    assert idx.tolist() == [2, 4]
    idx, _ = O.select_topk(s, 0, 2, 4)
    assert idx.tolist() == [1, 0, -1, -1]
    # independent library routine on a larger random case with many ties
    rng = np.random.default_rng(8)
    s = rng.integers(0, 20, 5000).astype(np.float32)
    import heapq

    want = heapq.nsmallest(100, range(10, 4990), key=lambda b: (-float(s[b]), b))
    assert O.select_topk(s, 10, 4990, 100)[0].tolist() == want


def check_attention_full_causal():
    """All blocks retrieved (or window covering all): full causal attention,
    against torch's scaled_dot_product_attention in float64."""
    rng = np.random.default_rng(9)
    for (N, B, S, W, n) in ((37, 4, 2, 5, 1), (64, 8, 0, 8, 6), (50, 50, 0, 50, 50), (33, 4, 1, 3, 3)):
        d = 16
        Q, K, V = rng.standard_normal((n, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))
        lo, hi = O.eligible_range(N, B, S, W)
        idx, _ = O.select_topk(rng.standard_normal(N // B + 1).astype(np.float32), lo, hi, N)
        T = O.attended_mask(N, B, S, W, idx)
        if N % B and N % B > W:
            continue  # an unattended tail: not the full-attention case
        assert T.all()
        got = O.attention(Q, K, V, T, 1 / math.sqrt(d))
        mask = torch.arange(N)[None, :] <= (N - n + torch.arange(n))[:, None]
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
            attn_mask=mask[None]).numpy()[0]
        assert np.max(np.abs(got - want)) < 1e-12


def check_attention_set_by_zero_query():
    """q = 0 gives equal weights, so the output is the plain mean of V over the
    attended set -- which pins the set itself (sinks, window, blocks, dedup,
    causal cut)."""
    rng = np.random.default_rng(10)
    for trial in range(40):
        N = int(rng.integers(20, 90))
        B = int(rng.integers(2, 12))
        S = int(rng.integers(0, 10))
        W = int(rng.integers(0, 20))
        n = int(rng.integers(1, 4))
        nb = N // B
        picks = sorted(set(rng.integers(0, max(nb, 1), 3).tolist())) if nb else []
        idx = np.array(picks + [-1], dtype=np.int32)
        V = rng.standard_normal((N, 3))
        T = O.attended_mask(N, B, S, W, idx)
        got = O.attention(np.zeros((n, 3)), rng.standard_normal((N, 3)), V, T, 0.5)
        for j in range(n):
            p = N - n + j
            toks = set(range(min(S, N))) | set(range(max(N - W, 0), N))
            for b in picks:
                toks |= set(range(b * B, (b + 1) * B))
            toks = sorted(t for t in toks if t <= p)
            assert np.allclose(got[j], V[toks].mean(axis=0), atol=1e-13, rtol=0), (trial, j)


def check_attention_skips_entries_outside_complete_blocks():
    """Entries that name no complete block add nothing: -1, negatives, indices
    past the memory, and nb itself when a partial tail block sits there
    outside the window (q = 0: the output is the mean of V over the set)."""
    rng = np.random.default_rng(12)
    N, B, S, W = 70, 8, 3, 4  # nb = 8, tail = tokens 64..69, window = 66..69
    V = rng.standard_normal((N, 2))
    K = rng.standard_normal((N, 2))
    for extra in ([8], [-1], [-5, 9], [8, 8, 1000]):
        idx = np.array([2, 5] + extra, dtype=np.int64)
        T = O.attended_mask(N, B, S, W, idx)
        toks = sorted(set(range(S)) | set(range(N - W, N)) | set(range(16, 24)) | set(range(40, 48)))
        assert np.flatnonzero(T).tolist() == toks, extra
        got = O.attention(np.zeros((1, 2)), K, V, T, 1.0)
        assert np.allclose(got[0], V[toks].mean(axis=0), atol=1e-14, rtol=0)


def check_attention_properties():
    rng = np.random.default_rng(11)
    N, B, d = 96, 8, 16
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    q = rng.standard_normal((1, d))
    idx = np.array([3, 7, 1, -1], dtype=np.int32)
    T = O.attended_mask(N, B, 2, 10, idx)
    base = O.attention(q, K, V, T, 0.25)
    # weights sum to one: V = 1 gives 1
    assert np.allclose(O.attention(q, K, np.ones((N, d)), T, 0.25), 1.0, atol=1e-14)
    # order of idx does not matter
    T2 = O.attended_mask(N, B, 2, 10, idx[[2, 0, 3, 1]])
    assert np.array_equal(O.attention(q, K, V, T2, 0.25), base)
    # the scale multiplies the logits
    assert np.allclose(O.attention(q * 0.25, K, V, T, 1.0), base, atol=1e-14)
    # output is a convex combination of the attended V rows
    assert np.all(base <= V[T].max(axis=0) + 1e-12) and np.all(base >= V[T].min(axis=0) - 1e-12)
    # shifting all logits equally leaves the output unchanged: add a constant
    # key component along a direction orthogonal-complemented by the query
    with pytest.raises(ValueError):
        O.attention(q, K, V, np.zeros(N, dtype=bool), 0.25)


def check_gqa_is_replicated_mha():
    rng = np.random.default_rng(12)
    Bt, Hq, Hkv, N, d, B = 2, 8, 2, 64, 8, 8
    q = rng.standard_normal((Bt, Hq, 1, d))
    K, V = rng.standard_normal((Bt, Hkv, N, d)), rng.standard_normal((Bt, Hkv, N, d))
    reps = np.stack([np.stack([O.reps_topnorm(K[b, g], B, 2) for g in range(Hkv)]) for b in range(Bt)])
    kw = dict(block=B, k=2, sinks=4, window=8, mode="topnorm")
    gqa = O.step(q, K, V, reps, **kw)
    G = Hq // Hkv
    rep = lambda X: np.repeat(X, G, axis=1)  # noqa: E731  (kv head g serves query heads gG..gG+G-1)
    mha = O.step(q, rep(K), rep(V), rep(reps), **kw)
    for key in gqa["out"]:
        assert np.array_equal(gqa["idx"][key], mha["idx"][key])
        assert np.array_equal(gqa["out"][key], mha["out"][key])
    assert O.kv_head_of(5, 32, 8) == 1 and O.kv_head_of(31, 32, 8) == 7 and O.kv_head_of(3, 4, 4) == 3


def check_planted_recall():
    """Blocks whose keys align with the query are retrieved (InfLLM's needle
    claim, here on synthetic planted blocks)."""
    from synth import WORKLOADS
    from synth import inputs as I

    w = WORKLOADS["infllm_gqa_decode_128k"].scaled(n_tokens=8192, window=512, sinks=128, n_q_heads=8,
                                                   n_kv_heads=2, k=10)
    x = I.make_all(w, "cpu")
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    K = f(x["k"])
    reps = np.stack([np.stack([O.reps_topnorm(K[b, g], w.block, w.reps_per_block)
                               for g in range(w.n_kv_heads)]) for b in range(w.batch)])
    res = O.step(f(x["q"]), K, f(x["v"]), reps, block=w.block, k=w.k, sinks=w.sinks,
                 window=w.window, mode="topnorm")
    for (b, h), blocks in x["planted"].items():
        assert set(blocks) <= set(res["idx"][(b, h)].tolist()), (h, blocks, res["idx"][(b, h)])


def check_hand_worked_fixture():
    """The hand-derived decode step in tests/golden/hand_worked_decode.json."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_decode.json")))
    K, V = np.array(g["K"], float), np.array(g["V"], float)
    assert O.eligible_range(g["N"], g["B"], g["S"], g["W"]) == tuple(g["eligible"])
    reps = O.reps_mean(K, g["B"], "f32")
    assert np.array_equal(reps[:, 0, :], np.array(g["reps"], float))
    lo, hi = g["eligible"]
    for j, qv in enumerate(g["q"]):
        q = np.array(qv, float)
        s = O.scores_dot_max(q, reps[lo:hi])
        assert s.tolist() == g["scores"][j]
        full = np.full(reps.shape[0], np.nan, dtype=np.float32)
        full[lo:hi] = s
        idx, _ = O.select_topk(full, lo, hi, g["k"])
        assert idx.tolist() == g["idx"][j]
        T = O.attended_mask(g["N"], g["B"], g["S"], g["W"], idx)
        out = O.attention(q[None], K, V, T, g["scale"])[0]
        assert np.allclose(out, g["out"][j], atol=1e-15, rtol=0)


def check_step_cosine_chunks():
    """Cosine mode selects per sequence, shared by all heads (MemLong 2.3.2):
    a stored chunk embedding equal to the query embedding wins, and every head
    attends the same chunks plus its causal local chunk."""
    rng = np.random.default_rng(13)
    Bt, H, n, d, C, nb = 1, 3, 4, 8, 4, 6           # 6 chunks of 4 tokens, last = current chunk
    N = nb * C
    E = rng.standard_normal((Bt, 1, nb, 1, 16))
    rq = E[:, 0, -1, 0, :].copy()
    E[0, 0, 2, 0, :] = 3.0 * rq[0]                   # chunk 2 points exactly along the query
    q = np.zeros((Bt, H, n, d))
    K, V = rng.standard_normal((Bt, H, N, d)), rng.standard_normal((Bt, H, N, d))
    res = O.step(q, K, V, E, block=C, k=2, sinks=0, window=C, mode="embed", rq=rq)
    idx = res["idx"][(0, 0)]
    assert idx[0] == 2 and len(res["idx"]) == 1
    for h in range(H):
        for j in range(n):
            toks = [t for b in idx for t in range(b * C, (b + 1) * C)] + list(range(N - C, N - C + j + 1))
            assert np.allclose(res["out"][(0, h)][j], V[0, h, toks].mean(axis=0), atol=1e-13)


def _tiny_attn_case(rng, n=3, N=11, d=5):
    Q = rng.normal(size=(n, d))
    K = rng.normal(size=(N, d))
    T = rng.random(N) < 0.7
    T[N - n:] = True  # every query sees at least its own token
    return Q, K, T


def check_weights_and_lse_library():
    """Weights are scipy's softmax of the visible logits (zero elsewhere); lse is scipy's logsumexp."""
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(71)
    for _ in range(20):
        Q, K, T = _tiny_attn_case(rng)
        n, N = Q.shape[0], K.shape[0]
        scale = float(rng.uniform(0.2, 1.5))
        P = O.attention_weights(Q, K, T, scale)
        L = O.attention_lse(Q, K, T, scale)
        for j in range(n):
            vis = [t for t in range(N) if T[t] and t <= N - n + j]
            z = scale * np.array([K[t] @ Q[j] for t in vis])
            want = np.zeros(N)
            want[vis] = softmax(z)
            assert np.allclose(P[j], want, atol=1e-15, rtol=1e-12)
            assert math.isclose(L[j], float(logsumexp(z)), rel_tol=1e-13, abs_tol=1e-13)
            # a weight is exp(logit - lse)
            assert np.allclose(P[j, vis], np.exp(z - L[j]), rtol=1e-12)


def check_window_mass_zero_query():
    """q = 0: every visible token weighs 1/|visible|, so the mass is a count (closed form)."""
    N, d, G, n, W = 13, 4, 3, 4, 7
    K = np.random.default_rng(5).normal(size=(N, d))
    T = np.zeros(N, dtype=bool)
    T[:2] = True
    T[N - W:] = True
    T[4:6] = True
    Qg = np.zeros((G, n, d))
    m = O.window_mass(Qg, K, T, 0.7, W)
    want = np.zeros(N)
    for j in range(n):
        vis = [t for t in range(N) if T[t] and t <= N - n + j]
        for t in vis:
            if t >= N - W:
                want[t] += G * Fraction(1, len(vis))
    assert np.allclose(m, want.astype(float), atol=1e-15)


def check_window_mass_conservation_and_range():
    """With the window over every token, the mass sums to heads x queries; outside the window it is 0."""
    rng = np.random.default_rng(9)
    G, n, N, d = 2, 3, 12, 4
    Qg = rng.normal(size=(G, n, d))
    K = rng.normal(size=(N, d))
    T = np.ones(N, dtype=bool)
    m = O.window_mass(Qg, K, T, 0.5, N)
    assert math.isclose(m.sum(), G * n, rel_tol=1e-13)
    assert (m > 0).all()
    W = 5
    mw = O.window_mass(Qg, K, T, 0.5, W)
    assert (mw[: N - W] == 0).all()
    assert np.allclose(mw[N - W:], m[N - W:], rtol=1e-14)
    # the last query's own token is seen by that query only
    Qa = rng.normal(size=(1, n, d))
    last = O.window_mass(Qa, K, T, 0.5, N)[N - 1]
    z = 0.5 * (K @ Qa[0, n - 1])
    assert math.isclose(last, math.exp(z[-1]) / np.exp(z).sum(), rel_tol=1e-12)


def check_reps_attnscore_bruteforce():
    """Largest mass first, ties to the lower token, keys copied; checked with an independent lexsort."""
    rng = np.random.default_rng(13)
    for _ in range(30):
        B, R, nb, d = 6, 3, 4, 3
        K = rng.normal(size=(nb * B, d))
        mass = rng.integers(0, 4, size=nb * B).astype(float)  # many ties
        blocks = [int(b) for b in rng.permutation(nb)[:3]]
        got = O.reps_attnscore(K, mass, B, R, blocks)
        for i, b in enumerate(blocks):
            toks = np.arange(b * B, (b + 1) * B)
            order = toks[np.lexsort((toks, -mass[toks]))][:R]
            assert np.array_equal(got[i], K[order])
    # one token far above the rest stands first
    K = np.arange(12.0).reshape(4, 3)
    mass = np.array([0.1, 5.0, 0.1, 0.2])
    got = O.reps_attnscore(K, mass, 4, 2, [0])
    assert np.array_equal(got[0], K[[1, 3]])


def check_count_hits_bincount():
    """Counts equal numpy's bincount over the valid entries (-1 and out-of-range skipped)."""
    rng = np.random.default_rng(21)
    for _ in range(20):
        nb = int(rng.integers(1, 40))
        h0 = rng.integers(0, 5, size=nb)
        idx = rng.integers(-3, nb + 3, size=int(rng.integers(0, 12)))
        got = O.count_hits(h0, idx, nb)
        ok = idx[(idx >= 0) & (idx < nb)]
        assert np.array_equal(got, h0 + np.bincount(ok, minlength=nb))


def _prune_case(rng):
    B = int(rng.integers(1, 9))
    nb = int(rng.integers(0, 60))
    tail = int(rng.integers(0, B))
    cap = int(rng.integers(nb * B + tail, 2 * (nb * B + tail) + 2 * B + 1))
    hits = rng.integers(0, 4, size=nb)
    return B, nb, tail, cap, hits


def check_prune_characterisation():
    """Oldest tenth gone, newest tenth kept, order kept, half the memory (or no middle left),
    and every evicted middle block ranks at or below every kept one by (hits, index)."""
    rng = np.random.default_rng(33)
    for _ in range(300):
        B, nb, tail, cap, hits = _prune_case(rng)
        plan = O.prune_plan(nb * B + tail, B, cap, hits)
        n10 = nb // 10
        assert (plan[:n10] == -1).all()
        assert (plan[nb - n10:] >= 0).all()
        kept = [b for b in range(nb) if plan[b] >= 0]
        assert [int(plan[b]) for b in kept] == list(range(len(kept)))
        mid = list(range(n10, nb - n10))
        kmid = [b for b in mid if plan[b] >= 0]
        emid = [b for b in mid if plan[b] < 0]
        if emid:
            assert len(kept) * B + tail <= cap // 2
            # one block fewer evicted would not fit
            assert (len(kept) + 1) * B + tail > cap // 2
        if kmid:
            assert (len(kept) * B + tail <= cap // 2) or not emid
        for e in emid:
            for k in kmid:
                assert (hits[e], e) < (hits[k], k)


def check_prune_equal_hits_and_tail():
    """Equal counts evict the oldest middle blocks first; the tail moves behind the kept blocks."""
    B, nb, tail, cap = 4, 40, 3, 200
    N = nb * B + tail
    plan = O.prune_plan(N, B, cap, np.zeros(nb, dtype=int))
    budget = (cap // 2 - tail) // B  # 24 blocks
    first = nb - budget
    assert (plan[:first] == -1).all() and list(plan[first:]) == list(range(budget))
    K = np.arange(N * 2, dtype=float).reshape(N, 2)
    assert np.array_equal(O.compact(K, plan, B, N), K[first * B:])
    # a hit on an old middle block saves it ahead of newer ones without hits
    hits = np.zeros(nb, dtype=int)
    hits[5] = 1
    plan2 = O.prune_plan(N, B, cap, hits)
    assert plan2[5] == 0 and plan2[first] == -1 and (plan2[first + 1:] >= 0).all()


def check_step_bruteforce():
    """One whole step on tiny inputs against pure-Python loops: the candidate
    blocks from their definition (complete, with a token outside the sinks and
    the window), each block's score as the largest dot with its representatives,
    its rank as a count of better candidates, and each query's output as a
    softmax written out over the union of sinks, window and chosen blocks that
    lies at or before the query's position (InfLLM "method"; Landmark Attention
    "proposed method")."""
    rng = np.random.default_rng(41)
    Hq, Hkv, N, B, R, d, n = 2, 1, 53, 5, 2, 4, 3
    for S, W, k in ((3, 7, 3), (6, 0, 2), (0, 11, 4), (2, 4, 20)):
        q = rng.standard_normal((1, Hq, n, d))
        K = rng.standard_normal((1, Hkv, N, d))
        V = rng.standard_normal((1, Hkv, N, d))
        reps = rng.standard_normal((1, Hkv, N // B, R, d))
        scale = 0.7
        res = O.step(q, K, V, reps, block=B, k=k, sinks=S, window=W, mode="given", scale=scale)
        cand = [b for b in range(N // B) if (b + 1) * B <= N
                and any(S <= t < N - W for t in range(b * B, (b + 1) * B))]
        for h in range(Hq):
            score = {}
            for b in cand:
                score[b] = np.float32(max(math.fsum(float(q[0, h, -1, i]) * float(reps[0, 0, b, r, i])
                                                     for i in range(d)) for r in range(R)))
            rank = {b: sum(1 for c in cand if score[c] > score[b] or (score[c] == score[b] and c < b))
                    for b in cand}
            chosen = sorted((b for b in cand if rank[b] < k), key=lambda b: rank[b])
            idx = res["idx"][(0, h)]
            assert [int(x) for x in idx if x >= 0] == chosen
            assert (idx[len(chosen):] == -1).all() and len(idx) == k
            T = set(range(min(S, N))) | set(range(max(N - W, 0), N))
            for b in chosen:
                T |= set(range(b * B, (b + 1) * B))
            for j in range(n):
                vis = sorted(t for t in T if t <= N - n + j)
                z = [scale * math.fsum(float(q[0, h, j, i]) * float(K[0, 0, t, i]) for i in range(d)) for t in vis]
                e = [math.exp(x) for x in z]
                den = math.fsum(e)
                for c in range(d):
                    want = math.fsum(e[m] * float(V[0, 0, t, c]) for m, t in enumerate(vis)) / den
                    assert abs(res["out"][(0, h)][j, c] - want) <= 1e-12


CHECKS = [check_round_f32, check_round_bf16, check_eligible_bruteforce, check_eligible_workloads,
          check_mean_exact, check_topnorm_bruteforce, check_dot_exact_mips, check_cosine,
          check_cosine_exact_rounding, check_group_max,
          check_topk_bruteforce, check_topk_ties_and_nan, check_attention_full_causal,
          check_attention_set_by_zero_query, check_attention_skips_entries_outside_complete_blocks,
          check_attention_properties, check_gqa_is_replicated_mha,
          check_planted_recall, check_hand_worked_fixture, check_step_cosine_chunks,
          check_weights_and_lse_library, check_window_mass_zero_query, check_window_mass_conservation_and_range,
          check_reps_attnscore_bruteforce, check_count_hits_bincount, check_prune_characterisation,
          check_prune_equal_hits_and_tail, check_step_bruteforce]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


# ---------------------------------------------------------------------------
# planted mistakes: every one must be caught by at least one check


def _mut_round_trunc(x, dtype):
    p, emin = O._FMT[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    e = np.maximum(e - 1, emin) - (p - 1)
    out[fin] = np.ldexp(np.trunc(np.ldexp(x[fin], -e)), e)
    return out


def _mut_round_half_up(x, dtype):
    p, emin = O._FMT[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    e = np.maximum(e - 1, emin) - (p - 1)
    out[fin] = np.ldexp(np.floor(np.ldexp(x[fin], -e) + 0.5), e)
    return out


def _mut_elig_floor(N, B, S, W):
    nb = N // B
    lo = min(S // B, nb)
    if N - W <= S:
        return lo, lo
    return lo, max(lo, min(nb, (N - W) // B))


def _mut_elig_no_guard(N, B, S, W):
    nb = N // B
    lo = min(S // B, nb)
    return lo, max(lo, min(nb, -(-(N - W) // B)))


def _mut_mean_div(K, B, dtype):
    nb = K.shape[0] // B
    s = K[: nb * B].reshape(nb, B, K.shape[1]).sum(axis=1)
    return O.round_to_dtype(s / max(B - 1, 1), dtype)[:, None, :]


def _mut_mean_unrounded(K, B, dtype):
    nb = K.shape[0] // B
    return (K[: nb * B].reshape(nb, B, K.shape[1]).sum(axis=1) / B)[:, None, :]


def _mut_topnorm_tie_high(K, B, R):
    nb = K.shape[0] // B
    out = np.empty((nb, R, K.shape[1]))
    for b in range(nb):
        blk = K[b * B:(b + 1) * B]
        n2 = (blk * blk).sum(axis=1)
        order = sorted(range(B), key=lambda t: (-n2[t], -t))
        out[b] = blk[order[:R]]
    return out


def _mut_topnorm_l1(K, B, R):
    nb = K.shape[0] // B
    out = np.empty((nb, R, K.shape[1]))
    for b in range(nb):
        blk = K[b * B:(b + 1) * B]
        n1 = np.abs(blk).sum(axis=1)
        order = sorted(range(B), key=lambda t: (-n1[t], t))
        out[b] = blk[order[:R]]
    return out


def _mut_dot_f32_accum(q, reps):
    return (reps.astype(np.float32) @ q.astype(np.float32)).max(axis=1).astype(np.float32)


def _mut_dot_mean_reps(q, reps):
    return (reps @ q).mean(axis=1).astype(np.float32)


def _mut_cos_no_qnorm(rq, E):
    ne = np.sqrt((E * E).sum(axis=1))
    s = np.zeros(E.shape[0])
    ok = ne != 0
    s[ok] = (E @ rq)[ok] / ne[ok]
    return s.astype(np.float32)


def _mut_cos_f64_norm_product(rq, E):
    # float64 formula with the norms multiplied after their square roots
    dot = E @ rq
    den = math.sqrt(float(rq @ rq)) * np.sqrt((E * E).sum(axis=1))
    s = np.zeros_like(dot)
    ok = den != 0
    s[ok] = dot[ok] / den[ok]
    return s.astype(np.float32)


def _mut_cos_f64_root_of_product(rq, E):
    # float64 formula with one square root of the product of the squared norms
    dot = E @ rq
    den = np.sqrt(float(rq @ rq) * (E * E).sum(axis=1))
    s = np.zeros_like(dot)
    ok = den != 0
    s[ok] = dot[ok] / den[ok]
    return s.astype(np.float32)


def _mut_group_mean(Qg, reps):
    dots = np.einsum("grd,hd->grh", reps, Qg)
    return dots.max(axis=1).mean(axis=1).astype(np.float32)


def _mut_group_first_head(Qg, reps):
    return O.scores_dot_max(Qg[0], reps)


def _mut_topk_tie_high(scores, lo, hi, k):
    def key(b):
        s = float(scores[b])
        return (1, 0.0, -b) if math.isnan(s) else (0, -s, -b)

    order = sorted(range(lo, hi), key=key)[:k]
    idx = np.full(k, -1, dtype=np.int32)
    vals = np.full(k, -np.inf, dtype=np.float32)
    idx[: len(order)] = order
    vals[: len(order)] = scores[order] if order else []
    return idx, vals


def _mut_topk_nan_first(scores, lo, hi, k):
    def key(b):
        s = float(scores[b])
        return (-1, 0.0, b) if math.isnan(s) else (0, -s, b)

    order = sorted(range(lo, hi), key=key)[:k]
    idx = np.full(k, -1, dtype=np.int32)
    vals = np.full(k, -np.inf, dtype=np.float32)
    idx[: len(order)] = order
    vals[: len(order)] = scores[order] if order else []
    return idx, vals


def _mut_mask_window_off_by_one(N, B, S, W, idx):
    T = np.zeros(N, dtype=bool)
    T[: min(S, N)] = True
    T[max(N - W + 1, 0):] = True
    for b in idx:
        if int(b) >= 0:
            T[int(b) * B: min((int(b) + 1) * B, N)] = True
    return T


def _mut_mask_block_short(N, B, S, W, idx):
    T = np.zeros(N, dtype=bool)
    T[: min(S, N)] = True
    T[max(N - W, 0):] = True
    for b in idx:
        if int(b) >= 0:
            T[int(b) * B: min((int(b) + 1) * B - 1, N)] = True
    return T


def _mut_mask_tail_entry(N, B, S, W, idx):
    # an entry equal to nb attends the partial tail block
    T = np.zeros(N, dtype=bool)
    T[: min(S, N)] = True
    T[max(N - W, 0):] = True
    for b in idx:
        if int(b) >= 0:
            T[int(b) * B: min((int(b) + 1) * B, N)] = True
    return T


def _mut_attention_no_causal(Q, K, V, T, scale):
    out = np.empty((Q.shape[0], V.shape[1]))
    for j in range(Q.shape[0]):
        if not T.any():
            raise ValueError
        z = scale * (K[T] @ Q[j])
        w = np.exp(z - z.max())
        out[j] = (w / w.sum()) @ V[T]
    return out


def _mut_attention_no_scale(Q, K, V, T, scale):
    return _orig_attention(Q, K, V, T, 1.0)


def _mut_attention_transposed(Q, K, V, T, scale):
    n, N = Q.shape[0], K.shape[0]
    out = np.empty((n, V.shape[1]))
    pos = np.arange(N)
    for j in range(n):
        sel = T & (pos <= N - n + j)
        if not sel.any():
            raise ValueError
        z = scale * (V[sel] @ Q[j])
        w = np.exp(z - z.max())
        out[j] = (w / w.sum()) @ K[sel]
    return out


def _mut_attention_query_first(Q, K, V, T, scale):
    n, N = Q.shape[0], K.shape[0]
    out = np.empty((n, V.shape[1]))
    pos = np.arange(N)
    for j in range(n):
        sel = T & (pos <= N - 1 - j)  # queries placed in reverse order
        if not sel.any():
            raise ValueError
        z = scale * (K[sel] @ Q[j])
        w = np.exp(z - z.max())
        out[j] = (w / w.sum()) @ V[sel]
    return out


def _mut_kv_head_mod(h, Hq, Hkv):
    return h % Hkv


def _mut_weights_no_causal(Q, K, T, scale):
    n, N = Q.shape[0], K.shape[0]
    P = np.zeros((n, N))
    for j in range(n):
        z = scale * (K[T] @ Q[j])
        w = np.exp(z - z.max())
        P[j, T] = w / w.sum()
    return P


def _mut_lse_log2(Q, K, T, scale):
    return _orig_lse(Q, K, T, scale) / math.log(2.0)


def _mut_mass_no_window(Qg, K, T, scale, W):
    return _orig_mass(Qg, K, T, scale, K.shape[0])


def _mut_mass_mean_heads(Qg, K, T, scale, W):
    return _orig_mass(Qg, K, T, scale, W) / Qg.shape[0]


def _mut_reps_attn_tie_high(K, mass, B, R, blocks):
    out = np.empty((len(blocks), R, K.shape[1]))
    for i, b in enumerate(blocks):
        order = sorted(range(b * B, (b + 1) * B), key=lambda t: (-mass[t], -t))
        out[i] = K[order[:R]]
    return out


def _mut_reps_attn_smallest(K, mass, B, R, blocks):
    out = np.empty((len(blocks), R, K.shape[1]))
    for i, b in enumerate(blocks):
        order = sorted(range(b * B, (b + 1) * B), key=lambda t: (mass[t], t))
        out[i] = K[order[:R]]
    return out


def _mut_hits_count_invalid(hits, idx, n_blocks):
    out = hits.copy()
    for b in idx:
        out[int(b) % n_blocks] += 1
    return out


def _mut_prune_tie_newer(n_tokens, B, capacity, hits):
    return _orig_prune(n_tokens, B, capacity, hits, key=lambda b: (int(hits[b]), -b))


def _mut_prune_most_hits(n_tokens, B, capacity, hits):
    return _orig_prune(n_tokens, B, capacity, hits, key=lambda b: (-int(hits[b]), b))


def _mut_prune_no_tail(n_tokens, B, capacity, hits):
    return _orig_prune((n_tokens // B) * B, B, capacity, hits)


_orig_attention = O.attention
_orig_lse = O.attention_lse
_orig_mass = O.window_mass


def _orig_prune(n_tokens, B, capacity, hits, key=None):
    # the oracle's plan with its eviction order replaced (for the planted mistakes)
    nb = n_tokens // B
    tail = n_tokens - nb * B
    n10 = nb // 10
    mid = list(range(n10, nb - n10))
    budget = max((capacity // 2 - tail) // B, 0)
    keep_mid = max(min(len(mid), budget - n10), 0)
    order = sorted(mid, key=key or (lambda b: (int(hits[b]), b)))
    evicted = set(order[: len(mid) - keep_mid]) | set(range(n10))
    new = np.full(nb, -1, dtype=np.int64)
    j = 0
    for b in range(nb):
        if b not in evicted:
            new[b] = j
            j += 1
    return new

_orig_step = O.step
_orig_compact = O.compact


def _mut_step_window_short(q, K, V, reps, **kw):
    return _orig_step(q, K, V, reps, **{**kw, "window": max(kw["window"] - 1, 0)})


def _mut_step_no_sinks(q, K, V, reps, **kw):
    return _orig_step(q, K, V, reps, **{**kw, "sinks": 0})


def _mut_step_k_short(q, K, V, reps, **kw):
    return _orig_step(q, K, V, reps, **{**kw, "k": max(kw["k"] - 1, 1)})


def _mut_step_unscaled(q, K, V, reps, **kw):
    return _orig_step(q, K, V, reps, **{**kw, "scale": 1.0})


def _mut_step_group_as_head(q, K, V, reps, **kw):
    return _orig_step(q, K, V, reps, **{**kw, "select": "head"})


def _mut_compact_no_tail(K, plan, B, n_tokens):
    return _orig_compact(K, plan, B, (n_tokens // B) * B)


def _mut_compact_reversed(K, plan, B, n_tokens):
    nb = n_tokens // B
    rows = [K[b * B:(b + 1) * B] for b in reversed(range(nb)) if plan[b] >= 0]
    rows.append(K[nb * B:n_tokens])
    return np.concatenate(rows, axis=0)


def _mut_compact_drops_first_kept(K, plan, B, n_tokens):
    nb = n_tokens // B
    rows = [K[b * B:(b + 1) * B] for b in range(nb) if plan[b] > 0]
    rows.append(K[nb * B:n_tokens])
    return np.concatenate(rows, axis=0)


MUTANTS = [
    ("step", _mut_step_window_short),
    ("step", _mut_step_no_sinks),
    ("step", _mut_step_k_short),
    ("step", _mut_step_unscaled),
    ("step", _mut_step_group_as_head),
    ("compact", _mut_compact_no_tail),
    ("compact", _mut_compact_reversed),
    ("compact", _mut_compact_drops_first_kept),
    ("round_to_dtype", _mut_round_trunc),
    ("round_to_dtype", _mut_round_half_up),
    ("eligible_range", _mut_elig_floor),
    ("eligible_range", _mut_elig_no_guard),
    ("reps_mean", _mut_mean_div),
    ("reps_mean", _mut_mean_unrounded),
    ("reps_topnorm", _mut_topnorm_tie_high),
    ("reps_topnorm", _mut_topnorm_l1),
    ("scores_dot_max", _mut_dot_f32_accum),
    ("scores_dot_max", _mut_dot_mean_reps),
    ("scores_group_max", _mut_group_mean),
    ("scores_group_max", _mut_group_first_head),
    ("scores_cosine", _mut_cos_no_qnorm),
    ("scores_cosine", _mut_cos_f64_norm_product),
    ("scores_cosine", _mut_cos_f64_root_of_product),
    ("select_topk", _mut_topk_tie_high),
    ("select_topk", _mut_topk_nan_first),
    ("attended_mask", _mut_mask_window_off_by_one),
    ("attended_mask", _mut_mask_block_short),
    ("attended_mask", _mut_mask_tail_entry),
    ("attention", _mut_attention_no_causal),
    ("attention", _mut_attention_no_scale),
    ("attention", _mut_attention_transposed),
    ("attention", _mut_attention_query_first),
    ("kv_head_of", _mut_kv_head_mod),
    ("attention_weights", _mut_weights_no_causal),
    ("attention_lse", _mut_lse_log2),
    ("window_mass", _mut_mass_no_window),
    ("window_mass", _mut_mass_mean_heads),
    ("reps_attnscore", _mut_reps_attn_tie_high),
    ("reps_attnscore", _mut_reps_attn_smallest),
    ("count_hits", _mut_hits_count_invalid),
    ("prune_plan", _mut_prune_tie_newer),
    ("prune_plan", _mut_prune_most_hits),
    ("prune_plan", _mut_prune_no_tail),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[f"{n}:{m.__name__}" for n, m in MUTANTS])
def test_planted_mistakes(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    caught = []
    for check in CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no check catches the planted mistake {mutant.__name__} in {name}"
