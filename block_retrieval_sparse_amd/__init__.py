"""Block-retrieval sparse attention for MI355X (gfx950).

Python face of libbrs: a KV memory with block representatives
(:class:`KVMemory`), block scoring, exact top-k selection and retrieval
attention.  Tensors are torch tensors on the GPU; every computation runs in
the library's HIP kernels on the current torch stream.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import BrsError, REP_MODES, check, lib

__all__ = ["KVMemory", "BlockCache", "select_topk", "BrsError", "lib", "version"]


def version() -> int:
    return lib.brs_version()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dt(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return _lib.BRS_F32
    if dtype == torch.bfloat16:
        return _lib.BRS_BF16
    raise TypeError(f"unsupported dtype {dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


class KVMemory:
    """One layer's block memory: K, V and per-block representatives.

    K and V are ``[batch][n_kv_heads][capacity][row_stride]``; reps are
    ``[batch][rep_heads][capacity // block][reps_per_block][rep_dim]``.
    With ``host=True`` K and V live in pinned host memory (the device reads
    and writes them directly; attention then goes through a
    :class:`BlockCache`), the representatives in device memory.
    """

    def __init__(self, batch: int, n_kv_heads: int, head_dim: int, capacity: int, block_size: int,
                 dtype: torch.dtype = torch.bfloat16, rep_mode: str = "mean", reps_per_block: int = 1,
                 rep_dim: int | None = None, rep_dtype: torch.dtype | None = None,
                 row_stride: int | None = None, device="cuda", host: bool = False):
        embed = rep_mode == "embed"
        rep_dim = rep_dim if rep_dim is not None else head_dim
        rep_dtype = rep_dtype if rep_dtype is not None else dtype
        row_stride = row_stride or head_dim
        rep_heads = 1 if embed else n_kv_heads
        if host:
            self.k = torch.zeros((batch, n_kv_heads, capacity, row_stride), dtype=dtype, pin_memory=True)
            self.v = torch.zeros((batch, n_kv_heads, capacity, row_stride), dtype=dtype, pin_memory=True)
        else:
            self.k = torch.zeros((batch, n_kv_heads, capacity, row_stride), dtype=dtype, device=device)
            self.v = torch.zeros_like(self.k)
        self.host = host
        self.device = torch.device(device)
        self.reps = torch.zeros((batch, rep_heads, capacity // block_size, reps_per_block, rep_dim),
                                dtype=rep_dtype, device=device)
        self.desc = _lib.brs_memory(
            dtype=_dt(dtype), batch=batch, n_kv_heads=n_kv_heads, head_dim=head_dim, row_stride=row_stride,
            block_size=block_size, reps_per_block=reps_per_block, rep_dim=rep_dim, rep_heads=rep_heads,
            rep_mode=REP_MODES[rep_mode], rep_dtype=_dt(rep_dtype), reserved=0, capacity=capacity, length=0,
            k=self.k.data_ptr(), v=self.v.data_ptr(), reps=self.reps.data_ptr())
        check(lib.brs_memory_check(self.desc))
        self.dtype, self.rep_mode, self.block_size = dtype, rep_mode, block_size
        self.batch, self.n_kv_heads, self.head_dim = batch, n_kv_heads, head_dim

    @property
    def length(self) -> int:
        return self.desc.length

    @property
    def n_blocks(self) -> int:
        return self.length // self.block_size

    @property
    def blocks_stride(self) -> int:
        return self.reps.shape[2]

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, reps_new: torch.Tensor | None = None,
               stream=None) -> None:
        """Append ``[batch][n_kv_heads][n][head_dim]`` K/V rows (contiguous)."""
        k_new, v_new = k_new.contiguous(), v_new.contiguous()
        if reps_new is not None:
            reps_new = reps_new.contiguous()
        n = k_new.shape[2]
        check(lib.brs_mem_append(self.desc, k_new.data_ptr(), v_new.data_ptr(), n, _ptr(reps_new),
                                 _stream(stream)))

    def eligible_range(self, n_sink: int, window: int) -> tuple[int, int]:
        lo, hi = _lib.c_int64(), _lib.c_int64()
        check(lib.brs_eligible_range(self.desc, n_sink, window, lo, hi))
        return lo.value, hi.value

    def score_blocks(self, qrep: torch.Tensor, lo: int, hi: int, scores: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
        """Dot-max scores ``[batch][Hq][blocks]`` from q ``[batch][Hq][d]``, or
        cosine scores ``[batch][1][blocks]`` from ``[batch][rep_dim]`` (embed mode)."""
        qrep = qrep.contiguous()
        hs = 1 if self.rep_mode == "embed" else qrep.shape[1]
        if scores is None:
            scores = torch.full((self.batch, hs, self.blocks_stride), float("nan"), dtype=torch.float32,
                                device=qrep.device)
        check(lib.brs_score_blocks(self.desc, qrep.data_ptr(), hs, lo, hi, scores.data_ptr(), _stream(stream)))
        return scores

    def workspace_bytes(self, n_q_heads: int, n_q: int, idx_heads: int, k: int, n_sink: int, window: int) -> int:
        n = _lib.c_size_t()
        check(lib.brs_attention_workspace_bytes(self.desc, n_q_heads, n_q, idx_heads, k, n_sink, window, n))
        return n.value

    def retrieval_attention(self, q: torch.Tensor, idx: torch.Tensor | None, n_sink: int, window: int,
                            scale: float | None = None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None,
                            lse: torch.Tensor | None = None) -> torch.Tensor:
        """q ``[batch][Hq][n_q][d]``, idx ``[batch][1 or Hq][k]`` int32 -> fp32 ``[batch][Hq][n_q][d]``;
        lse, if given, ``[batch][Hq][n_q]`` fp32 receives each query's log-sum-exp."""
        q = q.contiguous()
        bt, hq, n_q, d = q.shape
        if idx is None:
            idx_heads, k, iptr = 1, 0, None
        else:
            idx = idx.contiguous()
            idx_heads, k, iptr = idx.shape[1], idx.shape[2], idx.data_ptr()
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        nbytes = self.workspace_bytes(hq, n_q, idx_heads, k, n_sink, window)
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty((bt, hq, n_q, d), dtype=torch.float32, device=q.device)
        check(lib.brs_retrieval_attention(self.desc, q.data_ptr(), hq, n_q, iptr, idx_heads, k, n_sink, window,
                                          scale, out.data_ptr(), _ptr(lse), workspace.data_ptr(),
                                          workspace.numel(), _stream(stream)))
        return out

    def window_mass(self, q: torch.Tensor, lse: torch.Tensor, window: int, mass: torch.Tensor,
                    scale: float | None = None, stream=None) -> torch.Tensor:
        """Add the softmax weight every window token received from q (``[batch][Hq][n_q][d]``, with the
        log-sum-exp ``lse`` its attention call wrote) to ``mass`` ``[batch][n_kv_heads][capacity]`` fp32."""
        q = q.contiguous()
        bt, hq, n_q, d = q.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        check(lib.brs_window_mass(self.desc, q.data_ptr(), hq, n_q, lse.data_ptr(), window, scale, mass.data_ptr(),
                                  _stream(stream)))
        return mass

    def new_mass(self) -> torch.Tensor:
        """A zeroed attention-mass buffer ``[batch][n_kv_heads][capacity]`` fp32."""
        return torch.zeros((self.batch, self.n_kv_heads, self.k.shape[2]), dtype=torch.float32,
                           device=self.device)

    def new_hits(self) -> torch.Tensor:
        """A zeroed retrieval-count buffer ``[batch][capacity // block]`` int32."""
        return torch.zeros((self.batch, self.blocks_stride), dtype=torch.int32, device=self.device)

    def count_hits(self, idx: torch.Tensor, hits: torch.Tensor, stream=None) -> torch.Tensor:
        """Add one to ``hits`` for every valid entry of the selection ``idx`` ``[batch][heads][k]``."""
        idx = idx.contiguous()
        check(lib.brs_count_hits(self.desc, idx.data_ptr(), idx.shape[1], idx.shape[2], hits.data_ptr(),
                                 _stream(stream)))
        return hits

    def like(self) -> "KVMemory":
        """An empty memory with this one's geometry and buffers of its own."""
        d = self.desc
        return KVMemory(d.batch, d.n_kv_heads, d.head_dim, d.capacity, d.block_size, dtype=self.dtype,
                        rep_mode=self.rep_mode, reps_per_block=d.reps_per_block, rep_dim=d.rep_dim,
                        rep_dtype=self.reps.dtype, row_stride=d.row_stride, device=self.device, host=self.host)

    def prune_into(self, hits: torch.Tensor, dst: "KVMemory", dst_hits: torch.Tensor | None = None,
                   plan: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Copy what survives pruning into ``dst`` (see brs_mem_prune); returns the plan (new block
        index per old complete block, -1 if evicted)."""
        if plan is None:
            plan = torch.empty(self.blocks_stride, dtype=torch.int32, device=self.device)
        check(lib.brs_mem_prune(self.desc, hits.data_ptr(), dst.desc, _ptr(dst_hits), plan.data_ptr(),
                                _stream(stream)))
        return plan

    def reps_from_mass(self, mass: torch.Tensor, b0: int, b1: int, stream=None) -> None:
        """Build the representatives of blocks [b0, b1) from the accumulated mass (attnscore memories)."""
        check(lib.brs_reps_from_mass(self.desc, mass.data_ptr(), b0, b1, _stream(stream)))


class BlockCache:
    """A device cache of an offloaded memory's blocks: ``n_pages`` pages of
    ``block_size`` K/V rows per (batch, kv head) and the tables that map
    blocks to pages (see brs_cache_fetch)."""

    def __init__(self, mem: KVMemory, n_pages: int, stream=None):
        d = mem.desc
        dev = mem.device
        self.mem, self.n_pages = mem, n_pages
        self.k = torch.zeros((d.batch, d.n_kv_heads, n_pages * d.block_size, d.row_stride), dtype=mem.dtype,
                             device=dev)
        self.v = torch.zeros_like(self.k)
        bg = d.batch * d.n_kv_heads
        self.page_of_block = torch.empty((bg, d.capacity // d.block_size + 1), dtype=torch.int32, device=dev)
        self.page_block = torch.empty((bg, n_pages), dtype=torch.int32, device=dev)
        self.page_rows = torch.empty((bg, n_pages), dtype=torch.int32, device=dev)
        self.page_used = torch.empty((bg, n_pages), dtype=torch.int32, device=dev)
        self.fetched = torch.zeros((d.batch, d.n_kv_heads), dtype=torch.int32, device=dev)
        self.desc = _lib.brs_page_cache(k=self.k.data_ptr(), v=self.v.data_ptr(),
                                        page_of_block=self.page_of_block.data_ptr(),
                                        page_block=self.page_block.data_ptr(), page_rows=self.page_rows.data_ptr(),
                                        page_used=self.page_used.data_ptr(), n_pages=n_pages, reserved=0)
        self.steps = 0
        self.reset(stream)

    def reset(self, stream=None) -> None:
        check(lib.brs_cache_reset(self.mem.desc, self.desc, _stream(stream)))

    def fetch(self, idx: torch.Tensor | None, n_sink: int, window: int, stream=None) -> None:
        """Make resident every block an attention call with this selection reads."""
        self.steps += 1
        if idx is None:
            ih, k, ptr = 1, 0, None
        else:
            ih, k, ptr = idx.shape[1], idx.shape[2], idx.data_ptr()
        check(lib.brs_cache_fetch(self.mem.desc, self.desc, ptr, ih, k, n_sink, window, self.steps,
                                  self.fetched.data_ptr(), _stream(stream)))


def select_topk(scores: torch.Tensor, lo: int, hi: int, k: int, want_vals: bool = True, stream=None):
    """Top-k over columns [lo, hi) of ``[batch][heads][stride]`` fp32 scores.

    Returns (idx int32 ``[batch][heads][k]``, vals or None)."""
    bt, h, stride = scores.shape
    idx = torch.empty((bt, h, k), dtype=torch.int32, device=scores.device)
    vals = torch.empty((bt, h, k), dtype=torch.float32, device=scores.device) if want_vals else None
    check(lib.brs_select_topk(scores.data_ptr(), bt, h, stride, lo, hi, k, idx.data_ptr(), _ptr(vals),
                              _stream(stream)))
    return idx, vals
