"""brs_retrieval_step_static (workspace in a library-held device array, for
callers that cannot allocate) against brs_retrieval_step with a caller
workspace: identical selections, scores and outputs, on two calls in a row
with the second smaller than the first, through the C ABI."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from synth import WORKLOADS
from synth import inputs as I


def _desc(L, w, cap):
    return L.brs_memory(dtype=L.BRS_BF16, batch=w.batch, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                        row_stride=w.stride, block_size=w.block, reps_per_block=w.reps_per_block, rep_dim=w.rep_dim,
                        rep_heads=w.rep_heads, rep_mode=L.REP_MODES[w.rep_mode], rep_dtype=L.BRS_BF16, reserved=0,
                        capacity=cap, length=cap, k=0x10000, v=0x20000, reps=0x30000)


def test_static_step_rejects_oversized_workspace_on_host():
    """A step whose workspace exceeds the static array is refused before any device call."""
    from block_retrieval_sparse_amd import _lib as L

    w = WORKLOADS["retrievalattn_gqa_decode_1m_b8"]
    big = w.scaled(batch=64, k=2000)  # far more split-K partials than the array holds
    d = _desc(L, big, big.n_tokens)
    need = ctypes.c_size_t()
    rc = L.lib.brs_attention_workspace_bytes(d, big.n_q_heads, 1, big.n_q_heads, big.k, 0, 0, need)
    assert rc == 0 and need.value > L.lib.brs_static_scratch_bytes()
    rc = L.lib.brs_retrieval_step_static(d, 0x40000, big.n_q_heads, 1, 0x40000, big.n_q_heads, big.k, 0, 0, 0.1,
                                         0x50000, 0x60000, None, 0x70000, None, None)
    assert rc == -3 and b"static scratch" in L.lib.brs_last_error()


def _run(brs, L, w, static: bool):
    from block_retrieval_sparse_amd.pipeline import RetrievalStep

    x = I.make_all(w, "cuda")
    mem = brs.KVMemory(w.batch, w.n_kv_heads, w.head_dim, w.n_tokens, w.block, dtype=torch.bfloat16,
                       rep_mode=w.rep_mode, reps_per_block=w.reps_per_block, device="cuda")
    mem.append(x["k"], x["v"])
    st = RetrievalStep(mem, w.n_q_heads, 1, w.k, w.sinks, w.window)
    qrep = x["q"][:, :, -1, :].contiguous()
    if static:
        # the buffers a caller that cannot allocate would have set up beforehand
        st.scores.fill_(float("nan"))
        st.idx.fill_(-7)
        st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
        L.check(L.lib.brs_retrieval_step_static(mem.desc, x["q"].data_ptr(), w.n_q_heads, 1, qrep.data_ptr(),
                                                w.n_q_heads, w.k, w.sinks, w.window, st.scale, st.scores.data_ptr(),
                                                st.idx.data_ptr(), st.vals.data_ptr(), st.out.data_ptr(), None,
                                                stream))
    else:
        st.run(x["q"], qrep)
    torch.cuda.synchronize()
    return st.scores.cpu().numpy(), st.idx.cpu().numpy(), st.vals.cpu().numpy(), st.out.cpu().numpy(), (st.lo, st.hi)


@pytest.mark.gpu
def test_static_step_matches_workspace_step(gpu_lib):
    from block_retrieval_sparse_amd import _lib as L

    base = WORKLOADS["infllm_gqa_decode_128k"]
    calls = [base.scaled(n_tokens=16384 + 77, window=1024, sinks=64, k=24, planted_per_head=2, seed=4101),
             base.scaled(n_tokens=4096 + 13, window=256, sinks=16, k=6, n_q_heads=8, n_kv_heads=2,
                         planted_per_head=1, seed=4102)]
    for i, w in enumerate(calls):  # the second call is smaller than the first
        s_sc, s_idx, s_val, s_out, (lo, hi) = _run(gpu_lib, L, w, static=True)
        r_sc, r_idx, r_val, r_out, _ = _run(gpu_lib, L, w, static=False)
        assert np.array_equal(s_idx, r_idx), i
        assert np.array_equal(s_val, r_val), i
        assert np.array_equal(s_sc[:, :, lo:hi], r_sc[:, :, lo:hi]), i
        assert np.array_equal(s_out, r_out), i
        assert np.isfinite(s_out).all() and (s_idx >= 0).all(), i
