"""Tensors past 2^31 elements and 2^32 bytes (the 266304-token workload of
workloads.large_offsets: q, out, dout and dq are 4.36 GB each).  Rows from
token 262144 on sit past element 2^31, so any 32-bit element or byte offset
in the kernels, the scheduler or the zero fill would land them elsewhere.
The oracle recomputes whole (sequence, KV group) pairs at the start, just past
the boundary and in the last slot (which has padding rows); every row outside
a real range must be exactly +0.0 (LSE -inf) and no output may be non-finite.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_exact_zero_rows, assert_lse_close, f64, gpu_run, real_rows
import workloads

pytestmark = pytest.mark.gpu


def test_rows_past_element_2_31():
    case = workloads.large_offsets()
    T = case.q.shape[0]
    assert case.q.numel() > 2 ** 31 and case.q.numel() * case.q.element_size() > 2 ** 32
    o, l, dq, dk, dv = gpu_run(case)
    torch.cuda.synchronize()
    real = np.diff(case.cu_seqlens_q)
    pad = case.cu_seqlens_q_padded
    G = case.hq // case.hkv
    row_elems = case.hq * case.d
    first_far = next(b for b in range(case.batch) if int(pad[b]) * row_elems >= 2 ** 31)
    assert first_far == 256
    for b, g in [(0, 0), (first_far, 3), (case.batch - 1, case.hkv - 1)]:
        oq, L = int(pad[b]), int(real[b])
        hs = slice(g * G, (g + 1) * G)
        q = f64(case.q[oq:oq + L, hs])
        k = f64(case.k[oq:oq + L, g:g + 1])
        v = f64(case.v[oq:oq + L, g:g + 1])
        do = f64(case.dout[oq:oq + L, hs])
        ro, rl = oracle.attn_fwd_seq(q, k, v, case.scale, True)
        rdq, rdk, rdv = oracle.attn_bwd_seq(q, k, v, do, case.scale, True)
        rows = slice(oq, oq + L)
        assert_close(f"out[b{b},g{g}]", o[rows, hs], ro, case.dtype)
        assert_lse_close(l[rows, hs], rl, np.ones(L, bool))
        assert_close(f"dq[b{b},g{g}]", dq[rows, hs], rdq, case.dtype)
        assert_close(f"dk[b{b},g{g}]", dk[rows, g:g + 1], rdk, case.dtype)
        assert_close(f"dv[b{b},g{g}]", dv[rows, g:g + 1], rdv, case.dtype)
    outside = ~real_rows(case.cu_seqlens_q, pad, T)
    assert int(outside.sum()) == (1024 - 1000) + 64
    for name, t in (("out", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert_exact_zero_rows(name, t, outside)
        assert bool(torch.isfinite(t).all()), f"{name}: non-finite values"
    lo = l[torch.as_tensor(outside, device=l.device)]
    assert bool(torch.all(lo == -torch.inf))
