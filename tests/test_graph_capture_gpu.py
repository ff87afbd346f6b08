"""The forward and backward launch nothing but kernels on the caller's stream
(no allocation, no memset, no host synchronisation), so a step can be
captured into a HIP graph: every replay, with the program's own eager work
and synchronisations between replays, equals the eager call bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from helpers import cu_dev

pytestmark = pytest.mark.gpu


def test_fwd_bwd_graph_replays_equal_eager():
    import bwd_thd_varlen_amd as A
    A.lib()
    rng = np.random.default_rng(31)
    L, P = [300, 0, 129, 64], [320, 8, 136, 64]
    hq, hkv, d = 8, 2, 128
    T = sum(P)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16).cuda()
    q, k, v, do = mk(T, hq, d), mk(T, hkv, d), mk(T, hkv, d), mk(T, hq, d)
    cu = cu_dev(np.concatenate([[0], np.cumsum(L)]).astype(np.int32))
    cp = cu_dev(np.concatenate([[0], np.cumsum(P)]).astype(np.int32))
    ws = torch.empty(A.workspace_size(len(L), T, T, hq, hkv, d), dtype=torch.uint8, device="cuda")
    out, dq, dk, dv = (torch.empty_like(t) for t in (q, q, k, k))
    lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    kw = dict(cu_seqlens_q_padded=cp, cu_seqlens_kv_padded=cp, attn_mask_type="padding_causal",
              workspace=ws)

    def step():
        A.fwd(q, k, v, cu, cu, out=out, lse=lse, **kw)
        A.bwd(q, k, v, out, do, lse, cu, cu, dq=dq, dk=dk, dv=dv, **kw)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (out, lse, dq, dk, dv)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, lse, dq, dk, dv):   # poison the outputs between replays
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), want):
            assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32)), \
                f"replay {rep}: {name}"
