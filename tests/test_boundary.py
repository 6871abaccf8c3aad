"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/*.h declare, and rejects bad arguments on the host
before any device work; brs_eligible_range matches the oracle's brute force.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def L():
    from block_retrieval_sparse_amd import _lib

    return _lib


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(brs_\w+)\s*\(", text, flags=re.M)))


def test_header_declarations_are_exported(L):
    names = declared_functions()
    assert "brs_retrieval_attention" in names and len(names) >= 10
    for n in names:
        assert hasattr(L.lib, n), n
    assert sorted(L.EXPORTS) == names


def test_version(L):
    assert L.lib.brs_version() == 3


def desc(L, **kw):
    d = dict(dtype=L.BRS_BF16, batch=1, n_kv_heads=2, head_dim=128, row_stride=128, block_size=64,
             reps_per_block=1, rep_dim=128, rep_heads=2, rep_mode=L.REP_MEAN, rep_dtype=L.BRS_BF16, reserved=0,
             capacity=4096, length=4096, k=0x10000, v=0x20000, reps=0x30000)
    d.update(kw)
    return L.brs_memory(**d)


@pytest.mark.parametrize("bad", [
    dict(dtype=7), dict(rep_mode=9), dict(batch=0), dict(row_stride=64), dict(length=5000),
    dict(rep_heads=1), dict(rep_dim=64), dict(reps_per_block=2), dict(k=0), dict(v=0x20004),
    dict(reserved=1), dict(rep_mode=3, rep_heads=2), dict(capacity=1 << 40, length=0),
    dict(rep_mode=1, reps_per_block=100), dict(row_stride=127, head_dim=127, rep_dim=127),
])
def test_memory_check_rejects(L, bad):
    assert L.lib.brs_memory_check(desc(L, **bad)) == -1
    assert L.lib.brs_last_error()


def test_memory_check_accepts(L):
    assert L.lib.brs_memory_check(desc(L)) == 0
    assert L.lib.brs_memory_check(desc(L, rep_mode=L.REP_EMBED, rep_heads=1, rep_dim=768)) == 0
    assert L.lib.brs_memory_check(desc(L, rep_mode=L.REP_TOPNORM, reps_per_block=4)) == 0


def test_eligible_range_matches_oracle(L):
    import oracle.brs_oracle as O

    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    for N in (0, 1, 63, 64, 65, 500, 4096, 4100):
        for B in (1, 7, 64, 128):
            for S in (0, 4, 100, 5000):
                for Wn in (0, 1, 256, 4095, 10000):
                    m = desc(L, block_size=B, capacity=max(N, 1), length=N)
                    assert L.lib.brs_eligible_range(m, S, Wn, ctypes.byref(lo), ctypes.byref(hi)) == 0
                    assert (lo.value, hi.value) == O.eligible_range(N, B, S, Wn), (N, B, S, Wn)
    assert L.lib.brs_eligible_range(desc(L), -1, 0, ctypes.byref(lo), ctypes.byref(hi)) == -1


def test_append_rejects_before_device_work(L):
    m = desc(L, length=4000)
    assert L.lib.brs_mem_append(m, 0x1000, 0x2000, 97, None, None) == -2   # capacity
    assert m.length == 4000
    assert L.lib.brs_mem_append(m, 0x1000, 0x2000, -1, None, None) == -1
    assert L.lib.brs_mem_append(m, None, 0x2000, 5, None, None) == -1
    g = desc(L, rep_mode=L.REP_GIVEN, length=4000)
    assert L.lib.brs_mem_append(g, 0x1000, 0x2000, 90, None, None) == -1   # completes a block, no reps
    assert L.lib.brs_mem_append(m, 0x1000, 0x2000, 0, None, None) == 0     # no-op
    assert m.length == 4000


def test_score_select_attention_reject(L):
    m = desc(L)
    s = 0x40000
    assert L.lib.brs_score_blocks(m, 0x1000, 3, 0, 10, s, None) == -1          # heads not a multiple
    assert L.lib.brs_score_blocks(m, 0x1000, 4, 10, 5, s, None) == -1          # lo > hi
    assert L.lib.brs_score_blocks(m, 0x1000, 4, 0, 65, s, None) == -1          # beyond complete blocks
    e = desc(L, rep_mode=L.REP_EMBED, rep_heads=1, rep_dim=768)
    assert L.lib.brs_score_blocks(e, 0x1000, 2, 0, 10, s, None) == -1          # cosine has one head
    assert L.lib.brs_select_topk(s, 1, 4, 64, 0, 64, 0, 0x5000, None, None) == -3
    assert L.lib.brs_select_topk(s, 1, 4, 64, 0, 64, 4096, 0x5000, None, None) == -3
    assert L.lib.brs_select_topk(s, 1, 4, 64, 10, 5, 4, 0x5000, None, None) == -1
    assert L.lib.brs_select_topk(s, 1, 4, 64, 0, 65, 4, 0x5000, None, None) == -1
    n = ctypes.c_size_t()
    assert L.lib.brs_attention_workspace_bytes(m, 8, 1, 8, 32, 128, 1024, ctypes.byref(n)) == 0
    ws = n.value
    assert ws > 0
    assert L.lib.brs_attention_workspace_bytes(m, 8, 1, 8, 64, 128, 1024, ctypes.byref(n)) == 0
    assert n.value > 0
    assert L.lib.brs_attention_workspace_bytes(m, 8, 1, 8, 0, 0, 0, ctypes.byref(n)) == -5
    assert L.lib.brs_attention_workspace_bytes(m, 7, 1, 7, 4, 0, 0, ctypes.byref(n)) == -1
    args = dict(q=0x1000, hq=8, nq=1, idx=0x2000, ih=8, k=32, S=128, Wn=1024, sc=0.1, out=0x3000, lse=None)

    def call(ws_ptr=0x100000, ws_bytes=ws, **kw):
        a = dict(args)
        a.update(kw)
        return L.lib.brs_retrieval_attention(m, a["q"], a["hq"], a["nq"], a["idx"], a["ih"], a["k"], a["S"],
                                             a["Wn"], a["sc"], a["out"], a["lse"], ws_ptr, ws_bytes, None)

    assert call(hq=7) == -1
    assert call(ih=3) == -1
    assert call(nq=5000) == -1
    assert call(k=0, S=0, Wn=0) == -5
    assert call(ws_bytes=ws - 1) == -6
    assert call(ws_ptr=0x100010) == -6
    assert call(sc=float("inf")) == -1
    assert call(idx=None) == -1
    assert call(q=0x1004) == -1
    assert call(lse=0x7002) == -1                 # misaligned


def test_retrieval_step_rejects_before_device_work(L):
    m = desc(L)
    n = ctypes.c_size_t()
    assert L.lib.brs_attention_workspace_bytes(m, 8, 1, 8, 32, 128, 1024, ctypes.byref(n)) == 0
    ws = n.value
    args = dict(q=0x1000, hq=8, nq=1, qrep=0x4000, sh=8, k=32, S=128, Wn=1024, sc=0.1, scores=0x40000, idx=0x2000,
                vals=0x6000, out=0x3000, lse=None)

    def call(ws_ptr=0x100000, ws_bytes=ws, mem=m, **kw):
        a = dict(args)
        a.update(kw)
        return L.lib.brs_retrieval_step(mem, a["q"], a["hq"], a["nq"], a["qrep"], a["sh"], a["k"], a["S"], a["Wn"],
                                        a["sc"], a["scores"], a["idx"], a["vals"], a["out"], a["lse"], ws_ptr,
                                        ws_bytes, None)

    assert call(hq=7) == -1                       # not a multiple of the kv heads
    assert call(sh=4) == -1                       # neither the query heads nor the kv heads (2)
    assert call(sh=1) == -1                       # one list per sequence is for cosine scores
    assert call(nq=5000) == -1
    assert call(k=0, S=0, Wn=0) == -5             # nothing to attend
    assert call(k=4096) == -3                     # beyond the selection limit
    assert call(ws_bytes=ws - 1) == -6
    assert call(ws_ptr=0x100010) == -6
    assert call(qrep=None) == -1
    assert call(scores=None) == -1
    assert call(idx=None) == -1
    assert call(scores=0x40002) == -1             # misaligned
    assert call(sc=float("nan")) == -1
    assert call(mem=desc(L, reserved=1)) == -1
    assert call(S=-1) == -1
    e = desc(L, rep_mode=L.REP_EMBED, rep_heads=1, rep_dim=768)
    assert L.lib.brs_attention_workspace_bytes(e, 8, 1, 1, 32, 128, 1024, ctypes.byref(n)) == 0
    assert call(mem=e, ws_bytes=n.value, qrep=0x4001) == -1   # cosine query misaligned


def test_window_mass_and_reps_from_mass_reject_before_device_work(L):
    m = desc(L)
    wm = L.lib.brs_window_mass
    assert wm(m, 0x1000, 8, 1, 0x2000, 0, 0.1, 0x3000, None) == -1          # window < 1
    assert wm(m, 0x1000, 7, 1, 0x2000, 64, 0.1, 0x3000, None) == -1         # heads not a multiple of kv heads
    assert wm(m, 0x1000, 8, 0, 0x2000, 64, 0.1, 0x3000, None) == -1         # n_q < 1
    assert wm(m, None, 8, 1, 0x2000, 64, 0.1, 0x3000, None) == -1
    assert wm(m, 0x1000, 8, 1, None, 64, 0.1, 0x3000, None) == -1
    assert wm(m, 0x1000, 8, 1, 0x2000, 64, 0.1, 0x3002, None) == -1         # misaligned mass
    assert wm(m, 0x1000, 8, 1, 0x2000, 64, float("nan"), 0x3000, None) == -1
    rf = L.lib.brs_reps_from_mass
    assert rf(m, 0x3000, 0, 1, None) == -1                                  # not an ATTNSCORE memory
    a = desc(L, rep_mode=L.REP_ATTNSCORE, reps_per_block=4)
    assert L.lib.brs_memory_check(a) == 0
    nb = a.length // a.block_size
    assert rf(a, 0x3000, 0, nb + 1, None) == -1                             # past the complete blocks
    assert rf(a, 0x3000, 3, 2, None) == -1
    assert rf(a, None, 0, 1, None) == -1
    assert rf(a, 0x3000, 2, 2, None) == 0                                   # empty range: nothing to do
    assert L.lib.brs_memory_check(desc(L, rep_mode=L.REP_ATTNSCORE, reps_per_block=65)) == -1


def test_count_hits_and_prune_reject_before_device_work(L):
    m = desc(L)
    ch = L.lib.brs_count_hits
    assert ch(m, 0x1000, 0, 4, 0x2000, None) == -1          # idx_heads < 1
    assert ch(m, 0x1000, 2, -1, 0x2000, None) == -1         # k < 0
    assert ch(m, 0x1000, 2, 0, 0x2000, None) == 0           # nothing to count
    assert ch(m, None, 2, 4, 0x2000, None) == -1
    assert ch(m, 0x1000, 2, 4, 0x2002, None) == -1          # misaligned
    pr = L.lib.brs_mem_prune
    d = desc(L, k=0x90000, v=0xa0000, reps=0xb0000)
    assert pr(m, 0x1000, d, None, None, None) == -1         # no plan buffer
    assert pr(m, None, d, None, 0x3000, None) == -1         # no counts
    assert pr(m, 0x1000, desc(L, capacity=8192, k=0x90000, v=0xa0000, reps=0xb0000), None, 0x3000, None) == -1
    assert pr(m, 0x1000, desc(L, block_size=32, k=0x90000, v=0xa0000, reps=0xb0000), None, 0x3000, None) == -1
    assert pr(m, 0x1000, desc(L), None, 0x3000, None) == -1  # same buffers
    assert pr(m, 0x1000, None, None, 0x3000, None) == -1


def test_cache_calls_reject_before_device_work(L):
    m = desc(L, length=4096, capacity=8192)
    c = L.brs_page_cache(k=0x50000, v=0x60000, page_of_block=0x70000, page_block=0x71000, page_rows=0x72000,
                         page_used=0x73000, n_pages=20, reserved=0)
    # 4 query heads' lists over 2 kv heads: ceil(128 / 64) + 1024 / 64 + 2 lists * k = 2 + 16 + 2 * 2 = 22 > 20
    assert L.lib.brs_cache_fetch(m, c, 0x80000, 4, 2, 128, 1024, 1, None, None) == -2
    assert b"pages" in L.lib.brs_last_error()
    c.n_pages = 0
    assert L.lib.brs_cache_fetch(m, c, 0x80000, 2, 2, 128, 1024, 1, None, None) == -3
    c.n_pages = 64
    c.reserved = 1
    assert L.lib.brs_cache_reset(m, c, None) == -1
    c.reserved = 0
    c.k = 0x50008
    assert L.lib.brs_cache_reset(m, c, None) == -1     # misaligned pool
    c.k = 0x50000
    assert L.lib.brs_cache_fetch(m, c, 0x80000, 3, 2, 128, 1024, 1, None, None) == -1  # lists must tile the kv heads
    # a float32 memory is served by neither the slot-layout nor the prefill kernels, the two that read
    # K/V through a page table
    mf = desc(L, dtype=L.BRS_F32, rep_dtype=L.BRS_F32, length=4096, capacity=8192)
    n = ctypes.c_size_t()
    for n_q in (1, 64):
        assert L.lib.brs_attention_workspace_bytes(mf, 2, n_q, 2, 2, 128, 1024, ctypes.byref(n)) == 0
        assert L.lib.brs_retrieval_attention_cached(mf, c, 0x1000, 2, n_q, 0x80000, 2, 2, 128, 1024, 0.1, 0x3000,
                                                    None, 0x100000, n.value, None) == -3
        assert b"slot-layout and chunked-prefill" in L.lib.brs_last_error()


def test_measure_read_rejects_before_device_work(L):
    """The read-bandwidth reference validates its arguments on the host (fake
    device addresses: nothing is launched when a check fails)."""
    lib = L.lib
    f = lib.brs_measure_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32,
                  ctypes.c_void_p, ctypes.c_void_p]
    base, sink, offs = 0x10000, 0x20000, 0x30000
    inval = -1
    assert f(None, 1 << 20, None, 1, 0, sink, None) == inval          # no base
    assert f(base, 1 << 20, None, 1, 0, None, None) == inval          # no sink
    assert f(base, 8, None, 1, 0, sink, None) == inval                # under one 16-byte unit
    assert f(base, (1 << 20) + 8, None, 1, 0, sink, None) == inval    # not whole units
    assert f(base + 8, 1 << 20, None, 1, 0, sink, None) == inval      # misaligned base
    assert f(base, 1 << 20, None, 2, 0, sink, None) == inval          # a span is one chunk
    assert f(base, 1 << 31, offs, 4, 0, sink, None) == inval          # gathered chunks under 2^31 bytes
    assert f(base, 1 << 20, offs, 0, 0, sink, None) == inval          # no chunks
