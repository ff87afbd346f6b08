"""dK/dV of a GQA group spread over several workgroups per key tile: groups
of 8 or more query heads whose key tiles alone give few workgroups.  Each
workgroup walks a share of the group's query heads and writes fp32 partial
dK / dV planes, which a second kernel sums in a fixed order.  Parity with the
oracle in full (ragged sequences, all masks, head dims 32..256), with
dropout (exact gradients), an intermediate split on a larger problem, and
bitwise repeatability under a NaN-poisoned workspace.  The accumulating
chunked form is covered in tests/test_chunk_gpu.py."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_close, assert_lse_close, check_case, f64, gpu_run

pytestmark = pytest.mark.gpu


def split_of(batch, tq, tk, hq, hkv, d):
    """The number of workgroups per (key tile, KV head), read off the
    workspace size: only the partial planes (2 x split x tk x hkv x d fp32)
    grow with the head dim."""
    import bwd_thd_varlen_amd as A
    grow = A.workspace_size(batch, tq, tk, hq, hkv, d) - A.workspace_size(batch, tq, tk, hq, hkv, d - 8)
    return max(1, round(grow / (2 * tk * hkv * 8 * 4)))


def _case(lq, lk, pq, pk, hq, hkv, d, causal, dtype, seed):
    rng = np.random.default_rng(seed)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(td)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    tq, tk = int(sum(pq)) + 5, int(sum(pk)) + 5      # a few rows past every slot
    return workloads.Case(name="split_group", q=mk(tq, hq, d), k=mk(tk, hkv, d), v=mk(tk, hkv, d),
                          dout=mk(tq, hq, d), cu_seqlens_q=cu(lq), cu_seqlens_kv=cu(lk),
                          cu_seqlens_q_padded=cu(pq), cu_seqlens_kv_padded=cu(pk),
                          scale=d ** -0.5, causal=causal, dtype=dtype,
                          max_seqlen_q=int(max(pq)), max_seqlen_kv=int(max(pk)))


CASES = [  # (hq, hkv, d, causal, dtype)
    (16, 1, 128, True, "bf16"),
    (8, 1, 64, False, "fp16"),
    (16, 2, 256, True, "bf16"),
    (8, 1, 32, "bottom_right", "bf16"),
    (64, 8, 96, True, "fp16"),
    (8, 1, 80, "bottom_right", "bf16"),
    (16, 2, 160, False, "fp16"),
]


@pytest.mark.parametrize("hq,hkv,d,causal,dtype", CASES)
def test_split_group_parity(hq, hkv, d, causal, dtype):
    lq = [200, 0, 129, 64, 333]
    lk = [200, 40, 129, 64, 333] if causal is True else [150, 40, 200, 1, 300]
    pq = [208, 8, 136, 64, 340]
    pk = [208, 40, 136, 64, 333] if causal is True else [160, 40, 200, 8, 300]
    case = _case(lq, lk, pq, pk, hq, hkv, d, causal, dtype, seed=hq * 100 + d)
    split = split_of(case.batch, case.q.shape[0], case.k.shape[0], hq, hkv, d)
    assert 1 < split <= hq // hkv and (hq // hkv) % split == 0, split
    check_case(case)


def test_split_group_dropout_exact_gradients():
    from test_dropout_gpu import _case as drop_case, _gpu as drop_gpu, _oracle as drop_oracle
    from helpers import real_rows
    lq = [5, 130, 64, 0, 257, 33]
    lk = [5, 130, 64, 12, 257, 33]
    pq = [8, 130, 70, 4, 260, 40]
    pk = [9, 133, 64, 12, 300, 40]
    case = drop_case(lq, lk, pq, pk, hq=8, hkv=1, d=128, causal=True, dtype="bf16", seed=91)
    assert split_of(case.batch, case.q.shape[0], case.k.shape[0], 8, 1, 128) > 1
    drop = (0.2, 1234, 5)
    res, ref = drop_gpu(case, drop), drop_oracle(case, drop)
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
    assert_close("out", res[0], ref[0], "bf16", qrows)
    assert_lse_close(res[1], ref[1], qrows)
    assert_close("dq(exact)", res[2], ref[2], "bf16", qrows)
    assert_close("dk(exact)", res[3], ref[3], "bf16", krows)
    assert_close("dv(exact)", res[4], ref[4], "bf16", krows)


def test_intermediate_split_larger_problem():
    """8 sequences of 2048 tokens, 64 query heads on one KV head, d 128: the
    split (32) is below the group size (64); one whole sequence (all 64 heads)
    against the oracle."""
    L, B, hq, d = 2048, 8, 64, 128
    cu = np.arange(B + 1, dtype=np.int32) * L
    rng = np.random.default_rng(77)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
    T = B * L
    case = workloads.Case(name="mqa_16k", q=mk(T, hq, d), k=mk(T, 1, d), v=mk(T, 1, d),
                          dout=mk(T, hq, d), cu_seqlens_q=cu, cu_seqlens_kv=cu.copy(),
                          cu_seqlens_q_padded=cu.copy(), cu_seqlens_kv_padded=cu.copy(),
                          scale=d ** -0.5, causal=True, dtype="bf16", max_seqlen_q=L, max_seqlen_kv=L)
    split = split_of(B, T, T, hq, 1, d)
    assert split == 32, split
    o, l, dq, dk, dv = gpu_run(case)
    torch.cuda.synchronize()
    b = 5
    rows = slice(b * L, (b + 1) * L)
    q, k, v, do = (f64(t[rows]) for t in (case.q, case.k, case.v, case.dout))
    ro, rl = oracle.attn_fwd_seq(q, k, v, case.scale, True)
    rdq, rdk, rdv = oracle.attn_bwd_seq(q, k, v, do, case.scale, True)
    assert_close("out", o[rows], ro, "bf16")
    assert_lse_close(l[rows], rl, np.ones(L, bool))
    assert_close("dq", dq[rows], rdq, "bf16")
    assert_close("dk", dk[rows], rdk, "bf16")
    assert_close("dv", dv[rows], rdv, "bf16")


def test_split_group_bitwise_repeat():
    import bwd_thd_varlen_amd as A
    case = _case([300, 77, 129], [300, 77, 129], [320, 80, 136], [320, 80, 136], 16, 1, 128,
                 True, "bf16", seed=5)
    n = A.workspace_size(case.batch, case.q.shape[0], case.k.shape[0], 16, 1, 128)
    r1 = gpu_run(case)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")   # every float reads as NaN
    r2 = gpu_run(case, workspace=ws)
    for x, y in zip(r1, r2):
        assert torch.equal(x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32),
                           y.view(torch.int16) if y.element_size() == 2 else y.view(torch.int32))


def test_smaller_workspace_takes_a_smaller_split():
    """Fewer key tokens can mean more partial planes, so a workspace sized for
    a larger problem may be below workspace_size: the backward then halves the
    split until its planes fit (down to none) and the results stay at the
    bar; below the size without planes the call fails with EWORKSPACE."""
    import bwd_thd_varlen_amd as A
    from helpers import cu_dev, oracle_run, real_rows
    case = _case([200, 129, 64], [200, 129, 64], [208, 136, 64], [208, 136, 64], 16, 1, 128,
                 True, "bf16", seed=17)
    B, tq, tk = case.batch, case.q.shape[0], case.k.shape[0]
    assert split_of(B, tq, tk, 16, 1, 128) == 8      # a group of 16: at least 2 heads per workgroup
    base = A.workspace_size(B, tq, tk, 16, 16, 128)   # the same layout without planes (a group of 1)
    plane_pair = 2 * tk * 1 * 128 * 4                   # one dK and one dV plane
    ref = oracle_run(case)
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, tk, case.cu_seqlens_q)
    for nbytes in (base, base + 2 * plane_pair + 256):   # no split; room for split 2
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
        o, l, dq, dk, dv = gpu_run(case, workspace=ws)
        assert_close("dq", dq, ref[2], "bf16", qrows)
        assert_close("dk", dk, ref[3], "bf16", krows)
        assert_close("dv", dv, ref[4], "bf16", krows)
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, ck = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv)
    kw = dict(cu_seqlens_q_padded=cu_dev(case.cu_seqlens_q_padded),
              cu_seqlens_kv_padded=cu_dev(case.cu_seqlens_kv_padded), attn_mask_type="padding_causal")
    small = torch.empty(base - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(A.AttnError, match="WORKSPACE|workspace"):
        A.bwd(q, k, v, o, do, l, cq, ck, workspace=small, **kw)
