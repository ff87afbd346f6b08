"""Full-size parity of the benchmarked variant workloads, in the launch
configuration bench.py times: sbhd_65k (sbhd read in place), chunked_bottom_right
(bottom-right causal query chunks), chunks4_65k (four key chunks, merges and an
accumulating backward), dropout_65k (Philox keep mask) and fp8_65k (E4M3
inputs).  The GPU runs the whole workload; the oracle recomputes sampled
(sequence, KV group) pairs -- the shortest sequence in the first and last
groups and a longer one in a middle group -- and padding rows must be exact
zeros.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_lse_close, cu_dev, f64, real_rows
from oracle.fp8 import decode_e4m3
from oracle.philox import dropout_threshold, keep_mask
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def thr():
    return workloads.throughput_65k()


def _samples(case):
    """The shortest sequence in the first and last KV groups, and the fourth
    shortest (several key tiles, a ragged tail) in a middle group."""
    order = np.argsort(np.diff(case.cu_seqlens_q), kind="stable")
    return [(int(order[0]), 0), (int(order[0]), case.hkv - 1), (int(order[3]), case.hkv // 2)]


def _unit(case, b, g):
    """fp64 q, k, v, dout of sequence b, KV group g, and its query rows."""
    G = case.hq // case.hkv
    oq, L = int(case.cu_seqlens_q_padded[b]), int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])
    ok, Lk = int(case.cu_seqlens_kv_padded[b]), int(case.cu_seqlens_kv[b + 1] - case.cu_seqlens_kv[b])
    hs = slice(g * G, (g + 1) * G)
    return (f64(case.q[oq:oq + L, hs]), f64(case.k[ok:ok + Lk, g:g + 1]),
            f64(case.v[ok:ok + Lk, g:g + 1]), f64(case.dout[oq:oq + L, hs]),
            slice(oq, oq + L), slice(ok, ok + Lk), hs)


def _check_unit(name, case, res, b, g, keep=None, keep_scale=1.0):
    """Out, LSE, dQ, dK, dV of one (sequence, KV group) against the oracle.
    With dropout, dQ and dK are also held to the formula the kernels evaluate
    (P from the GPU's LSE, Delta from its O), as in the small dropout tests."""
    o, l, dq, dk, dv = res
    q, k, v, do, rq, rk, hs = _unit(case, b, g)
    ro, rl = oracle.attn_fwd_seq(q, k, v, case.scale, case.causal, keep=keep, keep_scale=keep_scale)
    rdq, rdk, rdv = oracle.attn_bwd_seq(q, k, v, do, case.scale, case.causal, keep=keep,
                                        keep_scale=keep_scale)
    tag = f"{name}[b{b},g{g}]"
    assert_close("out" + tag, o[rq, hs], ro, case.dtype)
    assert_lse_close(l[rq, hs], rl, np.ones(rq.stop - rq.start, bool))
    if keep is not None:
        fdq, fdk, _ = oracle.attn_bwd_seq(q, k, v, do, case.scale, case.causal, out=f64(o[rq, hs]),
                                          lse=f64(l[rq, hs]), mode="formula", keep=keep,
                                          keep_scale=keep_scale)
        assert_close("dq(formula)" + tag, dq[rq, hs], fdq, case.dtype)
        assert_close("dk(formula)" + tag, dk[rk, g:g + 1], fdk, case.dtype)
    assert_close("dq" + tag, dq[rq, hs], rdq, case.dtype)
    assert_close("dk" + tag, dk[rk, g:g + 1], rdk, case.dtype)
    assert_close("dv" + tag, dv[rk, g:g + 1], rdv, case.dtype)


def _padding_zero(case, res):
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, case.q.shape[0], case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, case.k.shape[0], case.cu_seqlens_q)
    for t, rows in ((res[0], qrows), (res[2], qrows), (res[3], krows), (res[4], krows)):
        sel = t[torch.as_tensor(~rows, device=t.device)]
        assert int(torch.count_nonzero(sel.view(torch.int16))) == 0


def _thd_run(case, **extra):
    import bwd_thd_varlen_amd as A
    print(f"[{case.name}] fwd+bwd at full size", flush=True)
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, ck = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv)
    kw = dict(cu_seqlens_q_padded=cu_dev(case.cu_seqlens_q_padded),
              cu_seqlens_kv_padded=cu_dev(case.cu_seqlens_kv_padded),
              max_seqlen_q=case.max_seqlen_q, max_seqlen_kv=case.max_seqlen_kv,
              attn_mask_type=case.mask_type, softmax_scale=case.scale, **extra)
    o, l = A.fwd(q, k, v, cq, ck, **kw)
    g = A.bwd(q, k, v, o, do, l, cq, ck, **kw)
    torch.cuda.synchronize()
    return (o, l) + tuple(g)


def test_sbhd_65k_sampled():
    import bwd_thd_varlen_amd as A
    case = workloads.sbhd_65k()
    S, B = case.max_seqlen_q, case.batch
    print("[sbhd_65k] fwd+bwd at full size", flush=True)
    sb = lambda t: t.cuda().view(B, S, *t.shape[1:]).transpose(0, 1).contiguous()
    q, k, v, do = sb(case.q), sb(case.k), sb(case.v), sb(case.dout)
    kw = dict(layout="sbhd", cu_seqlens_q=cu_dev(case.cu_seqlens_q),
              cu_seqlens_kv=cu_dev(case.cu_seqlens_kv), attn_mask_type=case.mask_type,
              softmax_scale=case.scale)
    o, l = A.fwd_batched(q, k, v, **kw)
    dq, dk, dv = A.bwd_batched(q, k, v, o, do, l, **kw)
    torch.cuda.synchronize()
    # back to THD rows b * S + i
    th = lambda t: t.transpose(0, 1).reshape(S * B, *t.shape[2:])
    res = (th(o), th(l), th(dq), th(dk), th(dv))
    for b, g in [(0, 0), (B - 1, case.hkv - 1), (B // 2, case.hkv // 2)]:
        _check_unit("sbhd", case, res, b, g)


def test_chunked_bottom_right_sampled():
    case = workloads.chunked_bottom_right()
    res = _thd_run(case)
    real_k = np.diff(case.cu_seqlens_kv)
    samples = [(int(np.argmin(real_k)), 0), (int(np.argmax(real_k)), case.hkv - 1),
               (int(np.argsort(real_k)[len(real_k) // 2]), case.hkv // 2)]
    for b, g in samples:
        _check_unit("br", case, res, b, g)
    _padding_zero(case, res)


def test_dropout_65k_sampled(thr):
    p, seed, offset = 0.1, 0x5EED, 0
    res = _thd_run(thr, dropout_p=p, rng_seed=seed, rng_offset=offset)
    t = dropout_threshold(p)
    G = thr.hq // thr.hkv
    for b, g in _samples(thr):
        L = int(thr.cu_seqlens_q[b + 1] - thr.cu_seqlens_q[b])
        keep = np.stack([keep_mask(L, L, b, h, thr.hq, seed, offset, t)
                         for h in range(g * G, (g + 1) * G)])
        _check_unit("dropout", thr, res, b, g, keep=keep, keep_scale=256.0 / (256.0 - t))
    _padding_zero(thr, res)


def test_chunks4_65k_sampled(thr):
    """Keys of every sequence in 4 chunks of consecutive positions: 4 chunk
    forwards with 3 merges, then 4 chunk backwards from the merged O / LSE with
    dQ accumulated; equal to the whole-sequence attention."""
    import bwd_thd_varlen_amd as A
    C = 4
    case = thr
    print("[chunks4_65k] chunk forwards, merges and backwards at full size", flush=True)
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, cqp = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_q_padded)
    real, offs = np.diff(case.cu_seqlens_kv), case.cu_seqlens_kv_padded[:-1]
    chunks = []
    for c in range(C):
        a, e = real * c // C, real * (c + 1) // C
        rows = np.concatenate([np.arange(o + x, o + y) for o, x, y in zip(offs, a, e)])
        idx = torch.as_tensor(rows, dtype=torch.long, device="cuda")
        chunks.append(dict(k=k.index_select(0, idx).contiguous(), v=v.index_select(0, idx).contiguous(),
                           cu=np.concatenate([[0], np.cumsum(e - a)]).astype(np.int32), pos=a))
    kw = dict(cu_seqlens_q_padded=cqp, attn_mask_type=case.mask_type, softmax_scale=case.scale)
    out = lse = None
    for c, ch in enumerate(chunks):
        o_c, l_c = A.fwd_chunk(q, ch["k"], ch["v"], cq, cu_dev(ch["cu"]),
                               kv_pos0=cu_dev(ch["pos"]), **kw)
        if c == 0:
            out, lse = o_c, l_c
        else:
            A.merge(out, lse, o_c, l_c)
    dq = torch.empty_like(q)
    for c, ch in enumerate(chunks):
        ch["dq"], ch["dk"], ch["dv"] = A.bwd_chunk(
            q, ch["k"], ch["v"], out, do, lse, cq, cu_dev(ch["cu"]), kv_pos0=cu_dev(ch["pos"]),
            dq=dq, accumulate={"dq"} if c > 0 else False, **kw)
    torch.cuda.synchronize()
    # dK / dV of each sequence back in its THD rows
    dk, dv = torch.zeros_like(k), torch.zeros_like(v)
    for c, ch in enumerate(chunks):
        a = real * c // C
        for b in range(case.batch):
            n = int(ch["cu"][b + 1] - ch["cu"][b])
            dst = slice(int(offs[b]) + int(a[b]), int(offs[b]) + int(a[b]) + n)
            dk[dst] = ch["dk"][int(ch["cu"][b]):int(ch["cu"][b]) + n]
            dv[dst] = ch["dv"][int(ch["cu"][b]):int(ch["cu"][b]) + n]
    res = (out, lse, dq, dk, dv)
    for b, g in _samples(case):
        _check_unit("chunks4", case, res, b, g)
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, case.q.shape[0])
    for t in (out, dq):
        assert int(torch.count_nonzero(t[torch.as_tensor(~qrows, device="cuda")].view(torch.int16))) == 0


def test_fp8_65k_sampled(thr):
    """The FP8 forward and backward (the fp8_65k and fp8_train_65k steps) at full size."""
    import bwd_thd_varlen_amd as A
    case = thr
    print("[fp8_65k] FP8-input forward at full size", flush=True)

    def quant(t):
        s = float(t.float().abs().max()) / 448.0
        return (t.cuda().float() / s).to(torch.float8_e4m3fn), s

    (q8, sq), (k8, sk), (v8, sv) = quant(case.q), quant(case.k), quant(case.v)
    o, l = A.fwd_fp8(q8, k8, v8, sq, sk, sv, cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv),
                     cu_dev(case.cu_seqlens_q_padded), cu_dev(case.cu_seqlens_kv_padded),
                     attn_mask_type=case.mask_type, softmax_scale=case.scale)
    torch.cuda.synchronize()
    # decoded codes of the sampled rows only
    dec = lambda t: decode_e4m3(t.view(torch.uint8).cpu().numpy())
    G = case.hq // case.hkv
    for b, g in _samples(case):
        oq = int(case.cu_seqlens_q_padded[b])
        L = int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])
        hs = slice(g * G, (g + 1) * G)
        ro, rl = oracle.attn_fwd_seq(dec(q8[oq:oq + L, hs]) * sq, dec(k8[oq:oq + L, g:g + 1]) * sk,
                                     dec(v8[oq:oq + L, g:g + 1]) * sv, case.scale, True)
        assert_close(f"out fp8[b{b},g{g}]", o[oq:oq + L, hs], ro, case.dtype)
        assert_lse_close(l[oq:oq + L, hs], rl, np.ones(L, bool))
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, case.q.shape[0])
    assert int(torch.count_nonzero(o[torch.as_tensor(~qrows, device="cuda")].view(torch.int16))) == 0

    # the FP8 backward of the fp8_train_65k step, from this forward's O and LSE
    print("[fp8_65k] FP8-input backward at full size", flush=True)
    dout = case.dout.cuda()
    dq, dk, dv = A.bwd_fp8(q8, k8, v8, sq, sk, sv, o, dout, l, cu_dev(case.cu_seqlens_q),
                           cu_dev(case.cu_seqlens_kv), cu_dev(case.cu_seqlens_q_padded),
                           cu_dev(case.cu_seqlens_kv_padded), attn_mask_type=case.mask_type,
                           softmax_scale=case.scale)
    torch.cuda.synchronize()
    for b, g in _samples(case):
        oq = int(case.cu_seqlens_q_padded[b])
        L = int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])
        hs = slice(g * G, (g + 1) * G)
        # self-attention workload: key rows share the query rows' offsets
        rdq, rdk, rdv = oracle.attn_bwd_seq(dec(q8[oq:oq + L, hs]) * sq,
                                            dec(k8[oq:oq + L, g:g + 1]) * sk,
                                            dec(v8[oq:oq + L, g:g + 1]) * sv,
                                            f64(case.dout[oq:oq + L, hs]), case.scale, True)
        assert_close(f"dq fp8[b{b},g{g}]", dq[oq:oq + L, hs], rdq, case.dtype)
        assert_close(f"dk fp8[b{b},g{g}]", dk[oq:oq + L, g:g + 1], rdk, case.dtype)
        assert_close(f"dv fp8[b{b},g{g}]", dv[oq:oq + L, g:g + 1], rdv, case.dtype)
    for t in (dq, dk, dv):
        assert int(torch.count_nonzero(t[torch.as_tensor(~qrows, device="cuda")].view(torch.int16))) == 0
