"""Every entry point that takes caller-allocated outputs rejects a wrong
output shape with AttnError before launching anything (the kernels write
through raw pointers and cannot catch an undersized tensor themselves)."""
import numpy as np
import pytest
import torch

from helpers import cu_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import bwd_thd_varlen_amd as A
    A.lib()
    return A


def _tensors(d=64, hq=4, hkv=2, T=24):
    g = torch.Generator().manual_seed(3)
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).cuda()
    cu = cu_dev(np.array([0, 10, T], np.int32))
    return mk(T, hq, d), mk(T, hkv, d), mk(T, hkv, d), mk(T, hq, d), cu


def test_thd_outputs(A):
    q, k, v, do, cu = _tensors()
    T, hq, d = q.shape
    small_q = torch.empty((T - 1, hq, d), dtype=q.dtype, device=q.device)
    small_k = torch.empty((T - 1, k.shape[1], d), dtype=q.dtype, device=q.device)
    small_lse = torch.empty((T, hq - 1), dtype=torch.float32, device=q.device)
    for kw in (dict(out=small_q), dict(lse=small_lse)):
        with pytest.raises(A.AttnError, match="shape"):
            A.fwd(q, k, v, cu, cu, **kw)
        with pytest.raises(A.AttnError, match="shape"):
            A.fwd_chunk(q, k, v, cu, cu, **kw)
    o, l = A.fwd(q, k, v, cu, cu)
    for kw in (dict(dq=small_q), dict(dk=small_k), dict(dv=small_k)):
        with pytest.raises(A.AttnError, match="shape"):
            A.bwd(q, k, v, o, do, l, cu, cu, **kw)
        with pytest.raises(A.AttnError, match="shape"):
            A.bwd_chunk(q, k, v, o, do, l, cu, cu, **kw)
        with pytest.raises(A.AttnError, match="shape"):
            A.bwd(q, k, v, o, do, l, cu, cu, dropout_p=0.1, rng_seed=1, **kw)
    torch.cuda.synchronize()


def test_batched_outputs(A):
    q, k, v, do, _ = _tensors(T=24)
    qb, kb, vb, dob = (t.view(2, 12, t.shape[1], t.shape[2]) for t in (q, k, v, do))
    o, l = A.fwd_batched(qb, kb, vb, layout="bshd")
    small = torch.empty((2, 11) + tuple(qb.shape[2:]), dtype=q.dtype, device=q.device)
    small_k = torch.empty((2, 11) + tuple(kb.shape[2:]), dtype=q.dtype, device=q.device)
    with pytest.raises(A.AttnError, match="shape"):
        A.fwd_batched(qb, kb, vb, layout="bshd", out=small)
    for kw in (dict(dq=small), dict(dk=small_k), dict(dv=small_k)):
        with pytest.raises(A.AttnError, match="shape"):
            A.bwd_batched(qb, kb, vb, o, dob, l, layout="bshd", **kw)
    torch.cuda.synchronize()


def test_fp8_outputs(A):
    q, k, v, do, cu = _tensors()
    q8, k8, v8 = (t.float().to(torch.float8_e4m3fn) for t in (q, k, v))
    T, hq, d = q.shape
    small = torch.empty((T - 1, hq, d), dtype=torch.bfloat16, device=q.device)
    small_k = torch.empty((T - 1, k.shape[1], d), dtype=torch.bfloat16, device=q.device)
    with pytest.raises(A.AttnError, match="shape"):
        A.fwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0, cu, cu, out=small)
    o, l = A.fwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0, cu, cu)
    for kw in (dict(dq=small), dict(dk=small_k), dict(dv=small_k)):
        with pytest.raises(A.AttnError, match="shape"):
            A.bwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0, o, do, l, cu, cu, **kw)
    torch.cuda.synchronize()
