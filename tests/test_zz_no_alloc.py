"""attn_bwd_thd_noalloc (the backward for callers that cannot allocate: its
scratch is the library's static per-GPU array) against attn_bwd_thd with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller problem, each bitwise equal to the workspace call (same kernels) and
so within the acceptance bar; outputs start as NaN so that an unwritten row
or a stale scratch entry would show."""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close, cu_dev, real_rows

pytestmark = pytest.mark.gpu


def _case(lq, lk, pq, pk, hq, hkv, d, causal, seed):
    rng = np.random.default_rng(seed)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    tq, tk = sum(pq), sum(pk)
    return workloads.Case(name="noalloc", q=mk(tq, hq, d), k=mk(tk, hkv, d), v=mk(tk, hkv, d),
                          dout=mk(tq, hq, d), cu_seqlens_q=cu(lq), cu_seqlens_kv=cu(lk),
                          cu_seqlens_q_padded=cu(pq), cu_seqlens_kv_padded=cu(pk),
                          scale=d ** -0.5, causal=causal, dtype="bf16")


def _both(A, case):
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, ck = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv)
    cqp, ckp = cu_dev(case.cu_seqlens_q_padded), cu_dev(case.cu_seqlens_kv_padded)
    kw = dict(cu_seqlens_q_padded=cqp, cu_seqlens_kv_padded=ckp, attn_mask_type=case.mask_type,
              softmax_scale=case.scale)
    o, l = A.fwd(q, k, v, cq, ck, **kw)
    ref = A.bwd(q, k, v, o, do, l, cq, ck, **kw)
    nan = lambda t: torch.full_like(t, float("nan"))
    dq, dk, dv = nan(q), nan(k), nan(k)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    st = A.attn_bwd_thd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), l.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cq.data_ptr(), ck.data_ptr(), cqp.data_ptr(),
        ckp.data_ptr(), case.batch, tq, tk, 0, 0, hq, hkv, d, case.scale,
        {"padding": 0, "padding_causal": 1}[case.mask_type], 0,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, A.status_string(st)
    torch.cuda.synchronize()
    return ref, (dq, dk, dv)


def test_noalloc_equals_workspace_call_twice_second_smaller():
    import bwd_thd_varlen_amd as A
    A.lib()
    big = _case([300, 0, 129, 64], [300, 40, 129, 64], [320, 8, 136, 64], [320, 40, 136, 64],
                hq=8, hkv=2, d=128, causal=True, seed=11)
    small = _case([50, 17], [50, 17], [56, 24], [56, 24], hq=4, hkv=1, d=64, causal=False,
                  seed=12)
    assert A.workspace_size(big.batch, big.q.shape[0], big.k.shape[0], 8, 2, 128) > \
        A.workspace_size(small.batch, small.q.shape[0], small.k.shape[0], 4, 1, 64)
    for case in (big, small):
        ref, got = _both(A, case)
        Tq, Tk = case.q.shape[0], case.k.shape[0]
        qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
        krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
        for name, r, g, rows in (("dq", ref[0], got[0], qrows), ("dk", ref[1], got[1], krows),
                                 ("dv", ref[2], got[2], krows)):
            assert torch.equal(r, g), f"{name}: not bitwise equal to attn_bwd_thd"
            assert_close(name, g, r.float().cpu().numpy(), "bf16", rows)


def test_noalloc_split_group_within_bar():
    """A group of 16 query heads on one KV head: attn_bwd_thd spreads the
    group over several dK/dV workgroups and sums their fp32 partials, while
    the no-allocation call (whose scratch holds no partial planes) keeps the
    group in one workgroup.  dQ is bitwise equal; dK / dV agree to the
    acceptance bar, and both sit within it of the oracle."""
    import bwd_thd_varlen_amd as A
    import oracle
    from helpers import f64
    A.lib()
    case = _case([200, 129, 64], [200, 129, 64], [208, 136, 64], [208, 136, 64],
                 hq=16, hkv=1, d=128, causal=True, seed=13)
    ref, got = _both(A, case)
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
    assert torch.equal(ref[0], got[0])
    args = (case.cu_seqlens_q, case.cu_seqlens_kv, case.cu_seqlens_q_padded, case.cu_seqlens_kv_padded)
    rdq, rdk, rdv = oracle.attn_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.dout), *args,
                                    scale=case.scale, causal=True)
    for name, r, g, o, rows in (("dk", ref[1], got[1], rdk, krows), ("dv", ref[2], got[2], rdv, krows)):
        assert_close(name + " (no-alloc vs split)", g, r.float().cpu().numpy(), "bf16", rows)
        assert_close(name + " (no-alloc vs oracle)", g, o, "bf16", rows)
        assert_close(name + " (split vs oracle)", r, o, "bf16", rows)


def test_noalloc_split_kernels_twice_second_smaller():
    """Head dims above 128 (the split dQ and dK/dV kernels, groups small
    enough that attn_bwd_thd does not spread them): bitwise equal to the
    workspace call, the second call on a smaller problem."""
    import bwd_thd_varlen_amd as A
    A.lib()
    big = _case([260, 1, 129], [260, 33, 129], [264, 8, 136], [264, 40, 136],
                hq=4, hkv=2, d=208, causal=False, seed=14)
    small = _case([70, 9], [70, 9], [72, 16], [72, 16], hq=2, hkv=1, d=160, causal=True, seed=15)
    for case in (big, small):
        ref, got = _both(A, case)
        for name, r, g in (("dq", ref[0], got[0]), ("dk", ref[1], got[1]), ("dv", ref[2], got[2])):
            assert torch.equal(r, g), f"{name} at d={case.d}: not bitwise equal to attn_bwd_thd"
