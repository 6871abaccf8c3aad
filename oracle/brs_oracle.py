"""CPU oracle for block-retrieval sparse attention (plain NumPy, float64).

THIS IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library never
calls it, links it or falls back to it, and it shares no code with the HIP
library: the two meet only in the seeded inputs of ``synth``.

What it computes, in the pages' order
-------------------------------------
The method shared by MemLong, InfLLM, Landmark Attention and
RetrievalAttention is: a long key/value memory cut into fixed-length blocks,
one or more representative vectors per block, a relevance score between the
query and each block's representatives, exact top-k block selection, and
softmax attention over the local context plus the selected blocks.

* O1 representatives (``reps_*``): block tiling from MemLong section 2.2.1
  (non-overlapping chunks) and Landmark Attention "proposed method"
  (fixed-length blocks); representative tokens from InfLLM "method" (a few
  tokens of each memory unit stand for it); given vectors from Landmark (one
  landmark key per block) and MemLong section 2.3.2 (the stored chunk
  embedding r^m = r^q).
* O2 eligibility (``eligible_range``): InfLLM "method" -- the memory holds
  what lies outside the local window.
* O3 scores (``scores_dot_max``, ``scores_group_max``, ``scores_cosine``):
  Landmark "proposed method" (similarity between the query and the landmark
  key), InfLLM "method" (block-level relevance), MemLong section 2.3.2
  (cosine similarity between r^q and the stored embeddings).
* O4 selection (``select_topk``): MemLong section 2.3.2 (TopK of the cosine
  scores, done with an exact index, section 2.4.2).
* O5 attended set (``attended_mask``): InfLLM "method" (local tokens plus a
  few relevant memory units), MemLong section 2.3.4 (retrieved chunks plus
  the current chunk), Landmark "proposed method" (a block's tokens are
  loaded only when its landmark is selected).
* O6 attention (``attention``): MemLong Figure 3 (local context is causal;
  retrieved chunks are visible in full), RetrievalAttention "proposed
  method" (exact attention over the tokens that matter).
* O7 attention-score representatives (``attention_weights``,
  ``attention_lse``, ``window_mass``, ``reps_attnscore``): InfLLM "method"
  (a memory unit's representative tokens are those that received the most
  attention in earlier attention computations).
* O8 retrieval counters and pruning (``count_hits``, ``prune_plan``,
  ``compact``): MemLong section 2.3.2, dynamic memory update.

Readings where the pages are silent (the same list is kept with the design
notes): attention sinks are the first S tokens; the window is the last W
tokens of memory; a partial tail block is never a candidate; a block wholly
inside sinks or window is not a candidate; ties go to the lower block index
and NaN ranks last; scores are exact-product float64 sums rounded once to
float32 (a cosine is the exact value rounded once); when the query heads of a
kv head share one selection, a block's score is the maximum over those heads
(as over a block's several representatives); softmax scale is 1/sqrt(d) and scores carry no scale; query head h
reads kv head h // G; several representatives combine by max; the selection
is per query head for dot scores and per sequence for cosine scores; local
and retrieved tokens share one softmax with no gate; query j of n sits at
position N - n + j; the cosine of a zero vector is 0; a token's attention
score for choosing representatives is the softmax weight it receives while
in the local window, summed over the query heads of its kv head and over
queries; a block's representatives are chosen when the block becomes a
candidate, from the mass accumulated up to then; a retrieval count is one per
selection-list entry (per query head for dot scores); pruning makes one
decision for the whole memory from the counts summed over its rows, with
10% = floor(nb / 10) blocks, 50% = capacity // 2 tokens, ties evicting the
older block, and the partial tail block always kept.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against brute force, exact rational arithmetic, closed forms or independent
library routines.  The pages print no worked numbers, so no value here is
pinned to a printed value.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------------------
# storage rounding


_FMT = {"f32": (24, -126), "bf16": (8, -126)}  # significand bits, min normal exponent


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest ``dtype`` value, ties to even.

    Plain definition of IEEE round-to-nearest-even with p significand bits:
    find the binade of |x| (clamped at the smallest normal binade so that
    subnormals get the fixed subnormal spacing), express x in units of that
    binade's spacing, round to the nearest integer with ties to even
    (``np.rint``), and scale back.  Results beyond the largest finite value
    become infinities.  Returns float64 holding exactly representable values.
    """
    p, emin = _FMT[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])            # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e - 1, emin)        # binade exponent, floor(log2|x|)
    spacing_exp = e - (p - 1)
    out[fin] = np.ldexp(np.rint(np.ldexp(x[fin], -spacing_exp)), spacing_exp)
    big = (2.0 - 2.0 ** (1 - p)) * 2.0 ** 127
    over = fin & (np.abs(np.where(fin, out, 0.0)) > big)
    out[over] = np.copysign(np.inf, x[over])
    return out


# ---------------------------------------------------------------------------
# O1: block representatives


def reps_mean(K: np.ndarray, B: int, dtype: str) -> np.ndarray:
    """Mean key of every complete block: [nb][1][d], rounded once to ``dtype``.

    K is one kv head's memory, [N][d] float64 holding the stored values.
    """
    nb = K.shape[0] // B
    d = K.shape[1]
    s = K[: nb * B].reshape(nb, B, d).sum(axis=1)
    return round_to_dtype(s / B, dtype)[:, None, :]


def reps_topnorm(K: np.ndarray, B: int, R: int) -> np.ndarray:
    """The R keys of every complete block with the largest L2 norm: [nb][R][d].

    Stand-in for InfLLM's representative tokens.  Squared norms are float64
    sums; order is (norm descending, token index ascending); the chosen keys
    are copied unchanged, in that order.
    """
    nb = K.shape[0] // B
    out = np.empty((nb, R, K.shape[1]))
    for b in range(nb):
        blk = K[b * B:(b + 1) * B]
        n2 = (blk * blk).sum(axis=1)
        order = sorted(range(B), key=lambda t: (-n2[t], t))
        out[b] = blk[order[:R]]
    return out


# ---------------------------------------------------------------------------
# O2: eligibility


def eligible_range(N: int, B: int, S: int, W: int) -> tuple[int, int]:
    """Candidate blocks [lo, hi): complete blocks with a token outside sinks and window.

    Tokens outside the sinks [0, S) and the window [N - W, N) are [S, N - W).
    Block b = [bB, bB + B) meets it iff b >= floor(S / B) and
    b < ceil((N - W) / B); it must also be complete, b < floor(N / B).
    """
    nb = N // B
    lo = min(S // B, nb)
    if N - W <= S:
        return lo, lo
    hi = min(nb, -(-(N - W) // B))
    return lo, max(lo, hi)


# ---------------------------------------------------------------------------
# O3: scores


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Query head h reads kv head floor(h / G), G = n_q_heads / n_kv_heads."""
    return h // (n_q_heads // n_kv_heads)


def scores_dot_max(q: np.ndarray, reps: np.ndarray) -> np.ndarray:
    """s_b = float32( max_r q . rep_{b,r} ) for one query head; q [d], reps [nb][R][d]."""
    dots = reps @ q                      # [nb][R], float64
    return dots.max(axis=1).astype(np.float32)


def _exact_ints(v: np.ndarray) -> list:
    """Every float64 of v as the exact integer v * 2**1074 (float64 values are
    integer multiples of 2**-1074)."""
    m, e = np.frexp(np.asarray(v, dtype=np.float64))
    mi = np.ldexp(m, 53).astype(np.int64)  # exact: m has 53 significant bits
    return [int(a) << int(b - 53 + 1074) if a >= 0 else -((-int(a)) << int(b - 53 + 1074))
            for a, b in zip(mi.tolist(), e.tolist())]


def _f32_nearest_signed_root(dot: int, prod: int) -> float:
    """The float32 nearest to dot / sqrt(prod) (prod > 0), ties to even.

    A float64 estimate fixes the neighbourhood; the choice between the
    estimate's float32 and its two neighbours is then made exactly, by
    comparing dot**2 with m**2 * prod for the midpoints m between them."""
    a2 = Fraction(dot * dot, prod)           # the exact square of the magnitude
    est = np.float32(math.sqrt(float(a2)))   # within a few float64 ulps of the magnitude
    lo_, hi_ = np.nextafter(est, np.float32(-np.inf)), np.nextafter(est, np.float32(np.inf))
    cands = [c for c in (lo_, est, hi_) if c >= 0]

    def above(mid: Fraction) -> int:        # sign of (magnitude - mid), exactly
        return (a2 > mid * mid) - (a2 < mid * mid)

    best = cands[0]
    for c0, c1 in zip(cands, cands[1:]):
        mid = (Fraction(float(c0)) + Fraction(float(c1))) / 2
        side = above(mid)
        if side > 0:
            best = c1
        elif side == 0:  # a tie: the even significand
            best = c0 if (int(np.float32(c0).view(np.uint32)) & 1) == 0 else c1
            break
        else:
            break
    return -float(best) if dot < 0 else float(best)


def scores_group_max(Qg: np.ndarray, reps: np.ndarray) -> np.ndarray:
    """One score per block for a whole group of query heads sharing a kv head:
    s_b = float32( max over the group's heads h and the block's reps r of
    q_h . rep_{b,r} ), exact products summed in float64; Qg [G][d], reps
    [nb][R][d].  A group that shares one selection ranks a block by its best
    match with any of its heads, the same way several representatives of a
    block combine (by max).  NaN in any head's dot makes the score NaN.
    """
    dots = np.einsum("grd,hd->grh", reps, Qg)  # [nb][R][G], float64
    return dots.reshape(dots.shape[0], -1).max(axis=1).astype(np.float32)


def scores_cosine(rq: np.ndarray, E: np.ndarray) -> np.ndarray:
    """s_b = float32( rq . e_b / (|rq| |e_b|) ), 0 when a norm is 0; E [nb][D].

    The cosine of the stored vectors is evaluated exactly (integer sums of
    exact products) and rounded once to the nearest float32, ties to even --
    the same single rounding the dot-product scores get."""
    q = _exact_ints(rq)
    qq = sum(x * x for x in q)
    out = np.zeros(E.shape[0], dtype=np.float32)
    for b in range(E.shape[0]):
        e = _exact_ints(E[b])
        dot = sum(x * y for x, y in zip(q, e))
        ee = sum(y * y for y in e)
        if qq == 0 or ee == 0 or dot == 0:
            continue
        out[b] = _f32_nearest_signed_root(dot, qq * ee)
    return out


# ---------------------------------------------------------------------------
# O4: top-k


def select_topk(scores: np.ndarray, lo: int, hi: int, k: int):
    """First min(k, hi - lo) candidates by (score descending, index ascending).

    NaN ranks after every number.  Returns (idx int32 [k], vals float32 [k]);
    unused slots hold -1 and -inf.
    """
    def key(b):
        s = float(scores[b])
        return (1, 0.0, b) if math.isnan(s) else (0, -s, b)

    order = sorted(range(lo, hi), key=key)[:k]
    idx = np.full(k, -1, dtype=np.int32)
    vals = np.full(k, -np.inf, dtype=np.float32)
    idx[: len(order)] = order
    vals[: len(order)] = scores[order] if order else []
    return idx, vals


# ---------------------------------------------------------------------------
# O5: attended token set


def attended_mask(N: int, B: int, S: int, W: int, idx) -> np.ndarray:
    """Boolean [N]: sinks [0, S), window [max(N - W, 0), N), and every selected block.

    A set: a token counted by several parts is still one token.  Only
    complete blocks can be selected (a partial tail block is never a
    candidate), so a selection entry outside [0, floor(N / B)) names no block
    and adds nothing -- -1 padding, and also an entry equal to the index of a
    partial tail block.
    """
    nb = N // B
    T = np.zeros(N, dtype=bool)
    T[: min(S, N)] = True
    T[max(N - W, 0):] = True
    for b in idx:
        b = int(b)
        if 0 <= b < nb:
            T[b * B:(b + 1) * B] = True
    return T


# ---------------------------------------------------------------------------
# O6: attention


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, T: np.ndarray, scale: float) -> np.ndarray:
    """Exact softmax attention of n queries over the set T, causal in position.

    Q [n][d], K and V [N][d] float64, T boolean [N].  Query j sits at
    position N - n + j and sees the tokens of T at or before it.  Softmax is
    computed with its maximum subtracted.  An empty set raises ValueError.
    """
    n, N = Q.shape[0], K.shape[0]
    out = np.empty((n, V.shape[1]))
    pos = np.arange(N)
    for j in range(n):
        sel = T & (pos <= N - n + j)
        if not sel.any():
            raise ValueError(f"query {j}: empty attended set")
        z = scale * (K[sel] @ Q[j])
        w = np.exp(z - z.max())
        out[j] = (w / w.sum()) @ V[sel]
    return out


# ---------------------------------------------------------------------------
# O7: attention mass of the window tokens, and representatives chosen by it
# (InfLLM "method": a memory unit is represented by its tokens that received
# the highest attention scores in earlier attention computations)


def attention_weights(Q: np.ndarray, K: np.ndarray, T: np.ndarray, scale: float) -> np.ndarray:
    """Softmax weights [n][N] of the attention in ``attention`` (0 off each query's visible set)."""
    n, N = Q.shape[0], K.shape[0]
    P = np.zeros((n, N))
    pos = np.arange(N)
    for j in range(n):
        sel = T & (pos <= N - n + j)
        if not sel.any():
            raise ValueError(f"query {j}: empty attended set")
        z = scale * (K[sel] @ Q[j])
        w = np.exp(z - z.max())
        P[j, sel] = w / w.sum()
    return P


def attention_lse(Q: np.ndarray, K: np.ndarray, T: np.ndarray, scale: float) -> np.ndarray:
    """Natural log of each query's softmax denominator: log of the sum of exp(scale q.k) over its visible set."""
    n, N = Q.shape[0], K.shape[0]
    out = np.empty(n)
    pos = np.arange(N)
    for j in range(n):
        sel = T & (pos <= N - n + j)
        if not sel.any():
            out[j] = -np.inf
            continue
        z = scale * (K[sel] @ Q[j])
        m = z.max()
        out[j] = m + math.log(np.exp(z - m).sum())
    return out


def window_mass(Qg: np.ndarray, K: np.ndarray, T: np.ndarray, scale: float, W: int) -> np.ndarray:
    """Attention that each token of the local window received in one call: [N].

    Qg [G][n][d] holds the query heads of one kv head.  The mass of token t is
    the sum, over those heads and the n queries, of its softmax weight; tokens
    before the window [N - W, N) get 0 (their memory units are already built).
    """
    N = K.shape[0]
    m = np.zeros(N)
    for h in range(Qg.shape[0]):
        m += attention_weights(Qg[h], K, T, scale).sum(axis=0)
    m[: max(N - W, 0)] = 0.0
    return m


def reps_attnscore(K: np.ndarray, mass: np.ndarray, B: int, R: int, blocks) -> np.ndarray:
    """For each listed block, its R keys with the largest accumulated mass: [len(blocks)][R][d].

    Order is (mass descending, token index ascending); the keys are copied
    unchanged, in that order.
    """
    out = np.empty((len(blocks), R, K.shape[1]))
    for i, b in enumerate(blocks):
        toks = range(b * B, (b + 1) * B)
        order = sorted(toks, key=lambda t: (-mass[t], t))
        out[i] = K[order[:R]]
    return out


# ---------------------------------------------------------------------------
# O8: retrieval counters and pruning (MemLong 2.3.2, dynamic memory update:
# on overflow keep the newest 10%, drop the oldest 10%, and evict the least
# retrieved of the middle 80% until half the memory is used)


def count_hits(hits: np.ndarray, idx: np.ndarray, n_blocks: int) -> np.ndarray:
    """Add one hit per valid entry of a selection list idx [k] to hits [n_blocks] (a copy is returned)."""
    out = hits.copy()
    for b in idx:
        b = int(b)
        if 0 <= b < n_blocks:
            out[b] += 1
    return out


def prune_plan(n_tokens: int, B: int, capacity: int, hits: np.ndarray) -> np.ndarray:
    """New block index of every complete block after pruning, -1 if evicted: [nb].

    nb = n_tokens // B complete blocks; the partial tail block is always kept,
    after them.  The oldest floor(nb / 10) blocks are dropped and the newest
    floor(nb / 10) kept; the middle blocks are evicted in order of (hits
    ascending, block index ascending) until the kept tokens (tail included)
    fit in capacity // 2, or no middle block is left.  Kept blocks keep their
    order.  ``hits`` [nb] are the retrieval counts summed over every row of
    the memory (one decision for the whole memory).
    """
    nb = n_tokens // B
    tail = n_tokens - nb * B
    n10 = nb // 10
    mid = list(range(n10, nb - n10))
    budget = max((capacity // 2 - tail) // B, 0)  # blocks that fit in half the memory
    keep_mid = max(min(len(mid), budget - n10), 0)
    order = sorted(mid, key=lambda b: (int(hits[b]), b))
    evicted = set(order[: len(mid) - keep_mid]) | set(range(n10))
    new = np.full(nb, -1, dtype=np.int64)
    j = 0
    for b in range(nb):
        if b not in evicted:
            new[b] = j
            j += 1
    return new


def compact(K: np.ndarray, plan: np.ndarray, B: int, n_tokens: int) -> np.ndarray:
    """Token rows [N'][...] after pruning: kept blocks in order, then the tail."""
    nb = n_tokens // B
    rows = [K[b * B:(b + 1) * B] for b in range(nb) if plan[b] >= 0]
    rows.append(K[nb * B:n_tokens])
    return np.concatenate(rows, axis=0)


# ---------------------------------------------------------------------------
# composition: one step over a whole workload


def build_reps(K_bg: np.ndarray, mode: str, B: int, R: int, dtype: str, given=None) -> np.ndarray:
    """O1 for one (batch, head): [nb][R][d]."""
    if mode == "mean":
        return reps_mean(K_bg, B, dtype)
    if mode == "topnorm":
        return reps_topnorm(K_bg, B, R)
    if mode in ("given", "embed"):
        return np.asarray(given, dtype=np.float64)
    raise ValueError(mode)


def step(q, K, V, reps, *, block: int, k: int, sinks: int, window: int, mode: str,
         rq=None, scale=None, heads=None, select: str = "head"):
    """One pass of the path (O3 -> O6) with representatives already built.

    q [β][Hq][n][d], K/V [β][Hkv][N][d], reps [β][Hr][nb][R][Dr] (all float64),
    rq [β][Dr] for cosine scoring.  ``heads`` limits the work to a list of
    (β, h) pairs.  ``select`` is "head" (one selection per query head) or
    "group" (one per kv head, shared by its query heads, from
    ``scores_group_max`` of their last queries); cosine scoring always makes
    one selection per sequence.  Returns dicts of scores, idx, vals and out:
    out keyed by (β, h); scores/idx/vals keyed by (β, h), (β, g) for group
    selection, or (β, 0) for cosine scoring.
    """
    Bt, Hq, n, d = q.shape
    Hkv, N = K.shape[1], K.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    lo, hi = eligible_range(N, block, sinks, window)
    nb_all = reps.shape[2]
    pairs = heads if heads is not None else [(b, h) for b in range(Bt) for h in range(Hq)]
    res = {"scores": {}, "idx": {}, "vals": {}, "out": {}, "range": (lo, hi)}
    for (b, h) in pairs:
        g = kv_head_of(h, Hq, Hkv)
        if mode == "embed":
            key = (b, 0)
            if key not in res["idx"]:
                s = np.full(nb_all, np.nan, dtype=np.float32)
                s[lo:hi] = scores_cosine(rq[b], reps[b, 0, lo:hi, 0, :])
                res["scores"][key] = s
                res["idx"][key], res["vals"][key] = select_topk(s, lo, hi, k)
        elif select == "group":
            key = (b, g)
            if key not in res["idx"]:
                G = Hq // Hkv
                s = np.full(nb_all, np.nan, dtype=np.float32)
                s[lo:hi] = scores_group_max(q[b, g * G:(g + 1) * G, -1], reps[b, g, lo:hi])
                res["scores"][key] = s
                res["idx"][key], res["vals"][key] = select_topk(s, lo, hi, k)
        else:
            key = (b, h)
            s = np.full(nb_all, np.nan, dtype=np.float32)
            s[lo:hi] = scores_dot_max(q[b, h, -1], reps[b, g, lo:hi])
            res["scores"][key] = s
            res["idx"][key], res["vals"][key] = select_topk(s, lo, hi, k)
        T = attended_mask(N, block, sinks, window, res["idx"][key])
        res["out"][(b, h)] = attention(q[b, h], K[b, g], V[b, g], T, scale)
    return res
