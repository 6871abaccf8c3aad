"""Workload table: the synthetic block-retrieval workloads, by shape only.

Each entry names what the workload stands in for on the pages:

* ``tiny_decode`` -- a small fp32 decode case (mean-of-block representatives).
* ``landmark_decode_32k`` -- Landmark Attention (method section: fixed-length
  blocks, one landmark key per block that decides retrieval), LLaMA-7B-like
  heads at a 32k context with 50-token blocks.
* ``infllm_gqa_decode_128k`` -- InfLLM (method section: sliding window plus
  block memory units, each represented by a few of its tokens), grouped-query
  decode at 131072 tokens with a 4K local window.
* ``memlong_chunk_prefill_80k`` -- MemLong (sections 2.3.2 and 2.3.4: cosine
  top-k over chunk embeddings, chunked long-input inference), OpenLLaMA-3B
  heads (H = 32, d = 100), 512-token chunks over an 80k-token memory.
* ``retrievalattn_gqa_decode_1m_b8`` -- RetrievalAttention (method section:
  out-of-distribution queries, a ~2% retrieval budget), batch 8 at 1M tokens.
* ``infllm_attnscore_decode_128k`` -- the InfLLM shape with representatives
  chosen by the attention the tokens received in the window (InfLLM method
  section) instead of by key norm.

No arithmetic of the method lives here; this module only fixes sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16": storage type of K, V, q
    n_tokens: int              # tokens in memory when the step runs
    block: int                 # tokens per block
    reps_per_block: int
    rep_mode: str              # "mean" | "topnorm" | "given" | "embed" | "attnscore"
    rep_dim: int
    k: int                     # blocks retrieved per score head
    window: int                # local window, last tokens of memory
    sinks: int                 # first tokens of memory, always attended
    n_q: int = 1               # queries per call (1 = decode)
    planted_per_head: int = 0  # blocks whose keys are 0.8 q_h + noise
    planted_scale: float = 0.8
    ood_offset: float = 0.0    # q = offset * u + N(0, I), u a random unit vector
    row_stride: int = 0        # elements per stored K/V row; 0 means head_dim
    seed: int = 1000

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def stride(self) -> int:
        return self.row_stride or self.head_dim

    @property
    def n_blocks(self) -> int:
        return self.n_tokens // self.block

    @property
    def rep_heads(self) -> int:
        return 1 if self.rep_mode == "embed" else self.n_kv_heads

    @property
    def score_heads(self) -> int:
        return 1 if self.rep_mode == "embed" else self.n_q_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "Workload":
        """Same structure, other sizes (used for oracle-sized parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_decode", batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
                 dtype="f32", n_tokens=4096, block=64, reps_per_block=1,
                 rep_mode="mean", rep_dim=64, k=4, window=256, sinks=4, seed=1001),
        Workload("landmark_decode_32k", batch=1, n_q_heads=32, n_kv_heads=32,
                 head_dim=128, dtype="bf16", n_tokens=32768, block=50,
                 reps_per_block=1, rep_mode="given", rep_dim=128, k=4, window=512,
                 sinks=0, seed=1002),
        Workload("infllm_gqa_decode_128k", batch=1, n_q_heads=32, n_kv_heads=8,
                 head_dim=128, dtype="bf16", n_tokens=131072, block=128,
                 reps_per_block=4, rep_mode="topnorm", rep_dim=128, k=32,
                 window=4096, sinks=128, planted_per_head=8, seed=1003),
        Workload("infllm_attnscore_decode_128k", batch=1, n_q_heads=32, n_kv_heads=8,
                 head_dim=128, dtype="bf16", n_tokens=131072, block=128,
                 reps_per_block=4, rep_mode="attnscore", rep_dim=128, k=32,
                 window=4096, sinks=128, planted_per_head=8, seed=1006),
        Workload("memlong_chunk_prefill_80k", batch=1, n_q_heads=32, n_kv_heads=32,
                 head_dim=100, dtype="bf16", n_tokens=81920 + 512, block=512,
                 reps_per_block=1, rep_mode="embed", rep_dim=768, k=5, window=512,
                 sinks=0, n_q=512, row_stride=104, seed=1004),
        Workload("retrievalattn_gqa_decode_1m_b8", batch=8, n_q_heads=32, n_kv_heads=8,
                 head_dim=128, dtype="bf16", n_tokens=1048576, block=64,
                 reps_per_block=1, rep_mode="mean", rep_dim=128, k=320, window=0,
                 sinks=0, ood_offset=2.0, seed=1005),
    ]
}

HEADLINE = "infllm_gqa_decode_128k"
