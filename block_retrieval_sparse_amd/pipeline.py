"""One retrieval-attention step over a KVMemory, with its buffers preallocated.

``RetrievalStep.run`` enqueues score_blocks -> select_topk ->
retrieval_attention on the current stream and returns the output tensor; no
allocation happens inside ``run``.
"""
from __future__ import annotations

import math

import torch

from . import BlockCache, KVMemory, _lib, _ptr, _stream, check, lib


class RetrievalStep:
    """``select``: "head" (one selection per query head) or "group" (one per kv
    head, shared by its query heads; dot scoring only).  Cosine scoring always
    makes one selection per sequence."""

    def __init__(self, mem: KVMemory, n_q_heads: int, n_q: int, k: int, n_sink: int, window: int,
                 scale: float | None = None, want_lse: bool = False, select: str = "head"):
        self.mem = mem
        self.n_q_heads, self.n_q, self.k = n_q_heads, n_q, k
        self.n_sink, self.window = n_sink, window
        self.scale = 1.0 / math.sqrt(mem.head_dim) if scale is None else scale
        dev = mem.device
        self.cosine = mem.rep_mode == "embed"
        if select not in ("head", "group"):
            raise ValueError("select must be 'head' or 'group'")
        self.grouped = select == "group" and not self.cosine
        self.score_heads = 1 if self.cosine else (mem.n_kv_heads if self.grouped else n_q_heads)
        self.scores = torch.full((mem.batch, self.score_heads, mem.blocks_stride), float("nan"),
                                 dtype=torch.float32, device=dev)
        self.idx = torch.full((mem.batch, self.score_heads, k), -1, dtype=torch.int32, device=dev)
        self.vals = torch.empty((mem.batch, self.score_heads, k), dtype=torch.float32, device=dev)
        self.out = torch.empty((mem.batch, n_q_heads, n_q, mem.head_dim), dtype=torch.float32, device=dev)
        # each query's log-sum-exp (needed to accumulate window attention mass)
        self.lse = torch.empty((mem.batch, n_q_heads, n_q), dtype=torch.float32, device=dev) if want_lse else None
        nbytes = mem.workspace_bytes(n_q_heads, n_q, self.score_heads, k, n_sink, window)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.lo, self.hi = mem.eligible_range(n_sink, window)

    def score(self, qrep: torch.Tensor, stream=None) -> None:
        if self.grouped:
            check(lib.brs_score_blocks_group(self.mem.desc, qrep.data_ptr(), self.n_q_heads, self.lo, self.hi,
                                             self.scores.data_ptr(), _stream(stream)))
            return
        check(lib.brs_score_blocks(self.mem.desc, qrep.data_ptr(), self.score_heads, self.lo, self.hi,
                                   self.scores.data_ptr(), _stream(stream)))

    def select(self, stream=None) -> None:
        if self.k == 0:
            return
        check(lib.brs_select_topk(self.scores.data_ptr(), self.mem.batch, self.score_heads, self.mem.blocks_stride,
                                  self.lo, self.hi, self.k, self.idx.data_ptr(), self.vals.data_ptr(),
                                  _stream(stream)))

    def attend(self, q: torch.Tensor, stream=None, profile_events=None) -> torch.Tensor:
        if profile_events is not None:
            check(lib.brs_profile_next_attention(profile_events[0], profile_events[1]))
        check(lib.brs_retrieval_attention(self.mem.desc, q.data_ptr(), self.n_q_heads, self.n_q,
                                          self.idx.data_ptr() if self.k else None, self.score_heads, self.k,
                                          self.n_sink, self.window, self.scale, self.out.data_ptr(),
                                          _ptr(self.lse), self.workspace.data_ptr(), self.workspace.numel(),
                                          _stream(stream)))
        return self.out

    def run(self, q: torch.Tensor, qrep: torch.Tensor | None = None, stream=None, profile_events=None):
        """One whole step in one library call (brs_retrieval_step).  q
        ``[batch][Hq][n_q][d]`` (contiguous); qrep is q's last query
        ``[batch][Hq][d]`` for dot scoring or the chunk embedding
        ``[batch][rep_dim]`` for cosine scoring."""
        if qrep is None:
            qrep = q[:, :, -1, :]
            if not qrep.is_contiguous():
                raise ValueError("pass a contiguous qrep")
        if profile_events is not None:
            check(lib.brs_profile_next_attention(profile_events[0], profile_events[1]))
        check(lib.brs_retrieval_step(self.mem.desc, q.data_ptr(), self.n_q_heads, self.n_q, qrep.data_ptr(),
                                     self.score_heads, self.k, self.n_sink, self.window, self.scale,
                                     self.scores.data_ptr(),
                                     self.idx.data_ptr(), self.vals.data_ptr(), self.out.data_ptr(),
                                     _ptr(self.lse), self.workspace.data_ptr(), self.workspace.numel(),
                                     _stream(stream)))
        return self.out

    def run_separate(self, q: torch.Tensor, qrep: torch.Tensor | None = None, stream=None, profile_events=None):
        """The same step as three calls: score_blocks, select_topk, retrieval_attention."""
        if qrep is None:
            qrep = q[:, :, -1, :]
            if not qrep.is_contiguous():
                raise ValueError("pass a contiguous qrep")
        self.score(qrep, stream)
        self.select(stream)
        return self.attend(q, stream, profile_events)


class CachedStep(RetrievalStep):
    """One step (decode, or a chunk of n_q queries) over an offloaded memory
    (K/V in host memory, see ``KVMemory(host=True)``): scores and selection
    as RetrievalStep, then brs_cache_fetch stages the blocks the step reads
    into the cache, then the attention reads them there
    (brs_retrieval_attention_cached).  Outputs are those of the same step on
    a resident memory, bit for bit."""

    def __init__(self, mem: KVMemory, cache: BlockCache, n_q_heads: int, k: int, n_sink: int, window: int,
                 scale: float | None = None, select: str = "head", n_q: int = 1):
        super().__init__(mem, n_q_heads, n_q, k, n_sink, window, scale=scale, select=select)
        self.cache = cache

    def fetch(self, stream=None) -> None:
        self.cache.fetch(self.idx if self.k else None, self.n_sink, self.window, stream)

    def attend(self, q: torch.Tensor, stream=None, profile_events=None) -> torch.Tensor:
        if profile_events is not None:
            check(lib.brs_profile_next_attention(profile_events[0], profile_events[1]))
        check(lib.brs_retrieval_attention_cached(self.mem.desc, self.cache.desc, q.data_ptr(), self.n_q_heads, self.n_q,
                                                 self.idx.data_ptr() if self.k else None, self.score_heads, self.k,
                                                 self.n_sink, self.window, self.scale, self.out.data_ptr(),
                                                 _ptr(self.lse), self.workspace.data_ptr(), self.workspace.numel(),
                                                 _stream(stream)))
        return self.out

    def run(self, q: torch.Tensor, qrep: torch.Tensor | None = None, stream=None, profile_events=None):
        if qrep is None:
            qrep = q[:, :, -1, :].contiguous()
        self.score(qrep, stream)
        self.select(stream)
        self.fetch(stream)
        return self.attend(q, stream, profile_events)


class AttnScoreMemory:
    """Decode loop state for attention-score representatives (InfLLM "method":
    a memory unit is represented by the tokens that received the most
    attention while they were in the local window).

    After each attention call (made with ``want_lse``), ``accumulate`` adds
    the window tokens' softmax weights to the mass buffer; ``refresh`` builds
    the representatives of the blocks that became candidates since the last
    refresh (their first token left the window), from the mass so far.
    """

    def __init__(self, mem: KVMemory, n_sink: int, window: int):
        if mem.rep_mode != "attnscore":
            raise ValueError("the memory's rep_mode must be 'attnscore'")
        self.mem, self.n_sink, self.window = mem, n_sink, window
        self.mass = mem.new_mass()
        self.built = mem.eligible_range(n_sink, window)[0]  # blocks below lo are never candidates

    def accumulate(self, q: torch.Tensor, lse: torch.Tensor, scale: float | None = None, stream=None) -> None:
        self.mem.window_mass(q, lse, self.window, self.mass, scale, stream)

    def refresh(self, stream=None) -> tuple[int, int]:
        """Build the representatives of newly eligible blocks; returns the block range built."""
        lo, hi = self.mem.eligible_range(self.n_sink, self.window)
        b0 = max(self.built, lo)
        if hi > b0:
            self.mem.reps_from_mass(self.mass, b0, hi, stream)
        self.built = max(self.built, hi)
        return b0, max(b0, hi)
