"""GPU parity of dropout (attn_fwd_thd_dropout / attn_bwd_thd_dropout).

The keep decision is integer work (a byte of a Philox word against a
threshold), so it is checked bit-exactly against the oracle's mask: with
V = identity rows the forward's O[i, j] is the dropped probability itself,
and with dO = identity rows the backward's dV[j, i] is; zeros must sit
exactly where the oracle drops (or masks) an element.  Values and gradients
then follow the usual bar against the oracle with the same (p, seed, offset):
every gradient against the exact one (definition mode), dQ and dK also
against the formula the kernels evaluate on the GPU forward's own O and LSE.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_lse_close, cu_dev, f64, real_rows
from oracle.philox import dropout_threshold
import workloads

pytestmark = pytest.mark.gpu


def _case(lq, lk, pq, pk, hq, hkv, d, causal, dtype, seed, q_scale=1.0):
    rng = np.random.default_rng(seed)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(td)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    tq, tk = sum(pq), sum(pk)
    q = (mk(tq, hq, d).float() * q_scale).to(td)
    return workloads.Case(name="dropout", q=q, k=mk(tk, hkv, d), v=mk(tk, hkv, d),
                          dout=mk(tq, hq, d), cu_seqlens_q=cu(lq), cu_seqlens_kv=cu(lk),
                          cu_seqlens_q_padded=cu(pq), cu_seqlens_kv_padded=cu(pk),
                          scale=1 / math.sqrt(d), causal=causal, dtype=dtype)


def _gpu(case, drop):
    import bwd_thd_varlen_amd as A
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, ck = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv)
    kw = dict(cu_seqlens_q_padded=cu_dev(case.cu_seqlens_q_padded),
              cu_seqlens_kv_padded=cu_dev(case.cu_seqlens_kv_padded),
              attn_mask_type=case.mask_type, softmax_scale=case.scale,
              dropout_p=drop[0], rng_seed=drop[1], rng_offset=drop[2])
    o, l = A.fwd(q, k, v, cq, ck, **kw)
    g = A.bwd(q, k, v, o, do, l, cq, ck, **kw)
    return (o, l) + tuple(g)


def _oracle(case, drop, **kw):
    args = (case.cu_seqlens_q, case.cu_seqlens_kv, case.cu_seqlens_q_padded,
            case.cu_seqlens_kv_padded)
    o, l = oracle.attn_fwd(f64(case.q), f64(case.k), f64(case.v), *args, scale=case.scale,
                           causal=case.causal, dropout=drop)
    g = oracle.attn_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.dout), *args,
                        scale=case.scale, causal=case.causal, dropout=drop, **kw)
    return (o, l) + tuple(g)


@pytest.mark.parametrize("causal", [False, True])
def test_keep_mask_bit_exact_forward_and_dkdv(causal):
    """O with V = identity rows and dV with dO = identity rows are the dropped
    probabilities: their zero patterns must equal the oracle's exactly."""
    L = [100, 37, 128]
    d, hq = 128, 4
    case = _case(L, L, L, L, hq=hq, hkv=2, d=d, causal=causal, dtype="bf16", seed=70,
                 q_scale=0.05)
    eye = torch.zeros(sum(L), 2, d, dtype=torch.bfloat16)
    deye = torch.zeros(sum(L), hq, d, dtype=torch.bfloat16)
    off = 0
    for n in L:
        eye[off:off + n, :, :n] = torch.eye(n, dtype=torch.bfloat16)[:, None, :]
        deye[off:off + n, :, :n] = torch.eye(n, dtype=torch.bfloat16)[:, None, :]
        off += n
    case.v, case.dout = eye, deye
    drop = (0.3, 0xDEADBEEF12345678, 5)
    o, l, dq, dk, dv = _gpu(case, drop)
    ro, rl, rdq, rdk, rdv = _oracle(case, drop)
    og, dvg = f64(o), f64(dv)
    assert np.array_equal(og == 0, ro == 0), "forward keep pattern differs"
    assert np.array_equal(dvg == 0, rdv == 0), "dK/dV keep pattern differs"
    assert_close("out", o, ro, "bf16")
    assert_close("dv", dv, rdv, "bf16")
    assert_close("dq", dq, rdq, "bf16")
    assert_close("dk", dk, rdk, "bf16")


@pytest.mark.parametrize("d,dtype,causal,p", [(64, "bf16", True, 0.1), (128, "bf16", False, 0.5),
                                              (128, "fp16", True, 0.2), (256, "bf16", True, 0.1),
                                              (32, "bf16", False, 0.3), (80, "fp16", True, 0.3),
                                              (192, "fp16", False, 0.2)])
def test_dropout_parity(d, dtype, causal, p):
    lq = [5, 130, 64, 0, 257, 33]
    lk = [5, 130, 64, 12, 257, 33] if causal else [9, 70, 64, 12, 300, 1]
    pq = [8, 130, 70, 4, 260, 40]
    pk = [9, 133, 64, 12, 300, 40]
    case = _case(lq, lk, pq, pk, hq=6, hkv=3, d=d, causal=causal, dtype=dtype, seed=71 + d)
    drop = (p, 42 + d, 3)
    res = _gpu(case, drop)
    ref = _oracle(case, drop)
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
    assert_close("out", res[0], ref[0], dtype, qrows)
    assert_lse_close(res[1], ref[1], qrows)
    # the backward from the GPU's own O: the formula the kernels evaluate
    form = _oracle(case, drop, out=f64(res[0]), lse=f64(res[1]), mode="formula")
    assert_close("dq", res[2], form[2], dtype, qrows)
    assert_close("dk", res[3], form[3], dtype, krows)
    assert_close("dv", res[4], form[4], dtype, krows)
    # and the exact gradient of the dropped attention (definition mode), so
    # that an error shared by the forward and the backward cannot pass
    assert_close("dq(exact)", res[2], ref[2], dtype, qrows)
    assert_close("dk(exact)", res[3], ref[3], dtype, krows)
    assert_close("dv(exact)", res[4], ref[4], dtype, krows)
    for name, t, rows in (("out", res[0], ~qrows), ("dq", res[2], ~qrows),
                          ("dk", res[3], ~krows), ("dv", res[4], ~krows)):
        assert torch.count_nonzero(t[torch.as_tensor(rows, device=t.device)].float()) == 0, name


def test_dropout_zero_equals_plain_and_repeats_bitwise():
    import bwd_thd_varlen_amd as A
    case = _case([77, 200], [77, 200], [80, 200], [80, 200], hq=8, hkv=2, d=128, causal=True,
                 dtype="bf16", seed=72)
    a = _gpu(case, (0.0, 1, 0))
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, ck = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv)
    kw = dict(cu_seqlens_q_padded=cu_dev(case.cu_seqlens_q_padded),
              cu_seqlens_kv_padded=cu_dev(case.cu_seqlens_kv_padded),
              attn_mask_type="padding_causal")
    o, l = A.fwd(q, k, v, cq, ck, **kw)
    b = (o, l) + tuple(A.bwd(q, k, v, o, do, l, cq, ck, **kw))
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    drop = (0.4, 99, 1)
    r1, r2 = _gpu(case, drop), _gpu(case, drop)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
    # another offset: another mask
    r3 = _gpu(case, (0.4, 99, 2))
    assert not torch.equal(r1[0], r3[0])
    assert dropout_threshold(0.4) == 102


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_dropout_bottom_right_unequal_lengths(dtype):
    """Dropout with the bottom-right causal mask: sequences with Lq < Lk, one
    with Lq > Lk (its first queries see no key: zero output, -inf LSE), an
    empty query side, and real != padded slots."""
    lq = [5, 130, 64, 0, 257, 33]
    lk = [40, 70, 200, 12, 300, 33]
    pq = [8, 130, 70, 4, 260, 40]
    pk = [40, 72, 200, 12, 300, 40]
    case = _case(lq, lk, pq, pk, hq=6, hkv=2, d=128, causal="bottom_right", dtype=dtype, seed=77)
    drop = (0.25, 0xC0FFEE, 7)
    res = _gpu(case, drop)
    ref = _oracle(case, drop)
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
    assert_close("out", res[0], ref[0], dtype, qrows)
    assert_lse_close(res[1], ref[1], qrows)
    form = _oracle(case, drop, out=f64(res[0]), lse=f64(res[1]), mode="formula")
    assert_close("dq", res[2], form[2], dtype, qrows)
    assert_close("dk", res[3], form[3], dtype, krows)
    assert_close("dq(exact)", res[2], ref[2], dtype, qrows)
    assert_close("dk(exact)", res[3], ref[3], dtype, krows)
    assert_close("dv", res[4], ref[4], dtype, krows)
