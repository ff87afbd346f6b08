"""GPU parity of the chunked (context-parallel) form: attn_fwd_thd_chunk,
attn_merge_thd and attn_bwd_thd_chunk.

Whole sequences are cut into uneven query and key chunks at per-sequence
positions; every chunk call is a THD call over the chunks of all sequences
(with padded slots).  The merged forward must match the oracle's attention
over the whole sequences, and the summed chunk backwards the oracle's
gradients from the same whole O and LSE.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import (assert_close, assert_lse_close, cu_dev, f64,
                     oracle_run)
import workloads

pytestmark = pytest.mark.gpu
PAD = 3   # padding rows appended to every chunk slot (filled with noise)


def _chunks(L, cuts):
    return [list(zip([0] + c, c + [n])) for n, c in zip(L, cuts)]


class ChunkCall:
    """The THD tensors of one chunk of every sequence (slot = chunk + PAD rows)."""

    def __init__(self, x_whole, offs, ranges, rng, td):
        pieces, real, self.rows = [], [], []
        for o, (a, b) in zip(offs, ranges):
            n = b - a
            pieces.append(x_whole[o + a:o + b])
            noise = torch.from_numpy(rng.standard_normal((PAD,) + tuple(x_whole.shape[1:]),
                                                         dtype=np.float32)).to(td)
            pieces.append(noise)
            real.append(n)
        self.x = torch.cat(pieces, 0)
        self.cu = np.concatenate([[0], np.cumsum(real)]).astype(np.int32)
        self.cu_pad = np.concatenate([[0], np.cumsum([n + PAD for n in real])]).astype(np.int32)
        self.pos0 = np.array([a for a, _ in ranges], np.int32)
        # (chunk row, whole row) pairs of the real tokens
        for b, (o, (a, e)) in enumerate(zip(offs, ranges)):
            self.rows += [(int(self.cu_pad[b]) + i, o + a + i) for i in range(e - a)]


def _run_chunked(L, qcuts, kcuts, hq, hkv, d, dtype, seed):
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(seed)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    T = sum(L)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(td)
    q, k, v, do = mk(T, hq, d), mk(T, hkv, d), mk(T, hkv, d), mk(T, hq, d)
    offs = np.concatenate([[0], np.cumsum(L)])[:-1]
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    case = workloads.Case(name="whole", q=q, k=k, v=v, dout=do, cu_seqlens_q=cu,
                          cu_seqlens_kv=cu.copy(), cu_seqlens_q_padded=cu.copy(),
                          cu_seqlens_kv_padded=cu.copy(), scale=1 / math.sqrt(d), causal=True,
                          dtype=dtype)
    qch, kch = _chunks(L, qcuts), _chunks(L, kcuts)
    nq, nk = max(map(len, qch)), max(map(len, kch))
    pick = lambda ch, i: [c[i] if i < len(c) else (c[-1][1], c[-1][1]) for c in ch]
    kcalls = []
    for ik in range(nk):
        kr = pick(kch, ik)
        kc, vc = ChunkCall(k, offs, kr, rng, td), ChunkCall(v, offs, kr, rng, td)
        kcalls.append((kc, vc))
    dev = "cuda"
    out_w = torch.zeros(T, hq, d, dtype=td, device=dev)
    lse_w = torch.full((T, hq), -math.inf, dtype=torch.float32, device=dev)
    dq_w = torch.zeros(T, hq, d, dtype=td, device=dev)
    dk_acc = [torch.zeros(kc.x.shape, dtype=td, device=dev) for kc, _ in kcalls]
    dv_acc = [torch.zeros(kc.x.shape, dtype=td, device=dev) for kc, _ in kcalls]
    qcalls = []
    for iq in range(nq):
        qr = pick(qch, iq)
        qc, doc = ChunkCall(q, offs, qr, rng, td), ChunkCall(do, offs, qr, rng, td)
        qcalls.append((qc, doc))
        kw = lambda kc: dict(cu_seqlens_q_padded=cu_dev(qc.cu_pad), cu_seqlens_kv_padded=cu_dev(kc.cu_pad),
                             q_pos0=cu_dev(qc.pos0), kv_pos0=cu_dev(kc.pos0),
                             attn_mask_type="padding_causal", softmax_scale=case.scale)
        qx = qc.x.cuda()
        acc_o = acc_l = None
        for kc, vc in kcalls:
            o_p, l_p = A.fwd_chunk(qx, kc.x.cuda(), vc.x.cuda(), cu_dev(qc.cu), cu_dev(kc.cu), **kw(kc))
            if acc_o is None:
                acc_o, acc_l = o_p, l_p
            else:
                A.merge(acc_o, acc_l, o_p, l_p)
        # padding rows of the chunk: +0.0 / -inf after every merge
        pad = np.ones(qc.x.shape[0], bool)
        pad[[r for r, _ in qc.rows]] = False
        assert int(torch.count_nonzero(acc_o[torch.as_tensor(pad, device=dev)].float())) == 0
        assert bool(torch.all(torch.isneginf(acc_l[torch.as_tensor(pad, device=dev)])))
        idx_c = torch.as_tensor([r for r, _ in qc.rows], dtype=torch.long, device=dev)
        idx_w = torch.as_tensor([w for _, w in qc.rows], dtype=torch.long, device=dev)
        out_w[idx_w] = acc_o[idx_c]
        lse_w[idx_w] = acc_l[idx_c]
        # backward of every pair from the whole (merged) O and LSE, accumulated
        dq_c = torch.zeros_like(qx)
        for j, (kc, vc) in enumerate(kcalls):
            A.bwd_chunk(qx, kc.x.cuda(), vc.x.cuda(), acc_o, doc.x.cuda(), acc_l, cu_dev(qc.cu),
                        cu_dev(kc.cu), dq=dq_c, dk=dk_acc[j], dv=dv_acc[j], accumulate=True,
                        **kw(kc))
        dq_w[idx_w] = dq_c[idx_c]
        assert int(torch.count_nonzero(dq_c[torch.as_tensor(pad, device=dev)].float())) == 0
    dk_w = torch.zeros(T, hkv, d, dtype=td, device=dev)
    dv_w = torch.zeros(T, hkv, d, dtype=td, device=dev)
    for j, (kc, _) in enumerate(kcalls):
        idx_c = torch.as_tensor([r for r, _ in kc.rows], dtype=torch.long, device=dev)
        idx_w = torch.as_tensor([w for _, w in kc.rows], dtype=torch.long, device=dev)
        dk_w[idx_w] = dk_acc[j][idx_c]
        dv_w[idx_w] = dv_acc[j][idx_c]
    return case, (out_w, lse_w, dq_w, dk_w, dv_w)


@pytest.mark.parametrize("d,dtype,hq,hkv", [(128, "bf16", 4, 2), (64, "fp16", 4, 2), (256, "bf16", 4, 2),
                                            (128, "bf16", 8, 1), (256, "fp16", 16, 2), (96, "bf16", 4, 2),
                                            (160, "fp16", 4, 2), (112, "bf16", 16, 2)])
def test_chunked_causal_matches_whole(d, dtype, hq, hkv):
    """Groups of 8 and more query heads take the split dK/dV (partial planes
    summed, then added into the accumulated dk / dv)."""
    L = [300, 77, 513, 1]
    qcuts = [[128, 200], [40], [100, 256, 400], []]
    kcuts = [[64, 150, 299], [5], [256], []]
    case, res = _run_chunked(L, qcuts, kcuts, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=50 + d + hq)
    o, l, dq, dk, dv = res
    ref_o, ref_l, *_ = oracle_run(case)
    rows = np.ones(case.q.shape[0], bool)
    assert_close("out", o, ref_o, dtype, rows)
    assert_lse_close(l, ref_l, rows)
    # gradients: the oracle's formula from the same whole O and LSE
    _, _, rdq, rdk, rdv = oracle_run(case, mode="formula", out=f64(o), lse=f64(l))
    assert_close("dq", dq, rdq, dtype, rows)
    assert_close("dk", dk, rdk, dtype, rows)
    assert_close("dv", dv, rdv, dtype, rows)


def test_chunk_calls_without_positions_equal_the_plain_calls_bitwise():
    """No positions, accumulate off: the chunk entry points are the plain calls."""
    import bwd_thd_varlen_amd as A
    L = [130, 64, 200]
    rng = np.random.default_rng(60)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16).cuda()
    T = sum(L) + 7
    q, k, v, do = mk(T, 8, 128), mk(T, 2, 128), mk(T, 2, 128), mk(T, 8, 128)
    cu = cu_dev(np.concatenate([[0], np.cumsum(L)]))
    for mask in ("padding", "padding_causal", "padding_causal_bottom_right"):
        o1, l1 = A.fwd(q, k, v, cu, cu, attn_mask_type=mask)
        o2, l2 = A.fwd_chunk(q, k, v, cu, cu, attn_mask_type=mask)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), mask
        g1 = A.bwd(q, k, v, o1, do, l1, cu, cu, attn_mask_type=mask)
        g2 = A.bwd_chunk(q, k, v, o1, do, l1, cu, cu, attn_mask_type=mask)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b), mask


def test_accumulate_adds_and_leaves_unreached_rows():
    """accumulate=True: out += share on reached rows; padding rows keep what they held."""
    import bwd_thd_varlen_amd as A
    L = [90, 0, 140]
    P = [96, 5, 150]
    rng = np.random.default_rng(61)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16).cuda()
    T = sum(P)
    q, k, v, do = mk(T, 4, 64), mk(T, 4, 64), mk(T, 4, 64), mk(T, 4, 64)
    cu = cu_dev(np.concatenate([[0], np.cumsum(L)]))
    cp = cu_dev(np.concatenate([[0], np.cumsum(P)]))
    kw = dict(cu_seqlens_q_padded=cp, cu_seqlens_kv_padded=cp, attn_mask_type="padding_causal")
    o, l = A.fwd(q, k, v, cu, cu, **kw)
    base = [mk(T, 4, 64) for _ in range(3)]          # arbitrary starting contents
    g = A.bwd(q, k, v, o, do, l, cu, cu, **kw)
    acc = [b.clone() for b in base]
    A.bwd_chunk(q, k, v, o, do, l, cu, cu, dq=acc[0], dk=acc[1], dv=acc[2], accumulate=True, **kw)
    real = np.zeros(T, bool)
    for o_, n in zip(np.concatenate([[0], np.cumsum(P)])[:-1], L):
        real[o_:o_ + n] = True
    rt = torch.as_tensor(real, device="cuda")
    for name, a, b0, gi in zip(("dq", "dk", "dv"), acc, base, g):
        assert torch.equal(a[~rt], b0[~rt]), f"{name}: unreached rows changed"
        want = (b0.float() + gi.float()).to(torch.bfloat16)   # one rounding of the fp32 sum
        diff = (a[rt].float() - want[rt].float()).abs().max().item()
        ulp = want[rt].float().abs().max().item() * 2.0 ** -7
        assert diff <= ulp, f"{name}: {diff} > {ulp}"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_merge_kernel_against_oracle(dtype):
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(62)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    T, H, d = 333, 6, 48
    oa = torch.from_numpy(rng.standard_normal((T, H, d), dtype=np.float32)).to(td)
    ob = torch.from_numpy(rng.standard_normal((T, H, d), dtype=np.float32)).to(td)
    la = torch.from_numpy((rng.standard_normal((T, H)) * 4).astype(np.float32))
    lb = torch.from_numpy((rng.standard_normal((T, H)) * 4).astype(np.float32))
    la[::7] = -math.inf                      # empty first side
    lb[::5] = -math.inf                      # empty second side (both on rows % 35 == 0)
    ro, rl = oracle.merge_partials(f64(oa), f64(la), f64(ob), f64(lb))
    o, l = oa.cuda(), la.cuda()
    A.merge(o, l, ob.cuda(), lb.cuda())
    lg = f64(l)
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.all(np.abs(lg[fin] - rl[fin]) <= 1e-5 * (1 + np.abs(rl[fin])))
    og = f64(o)
    both_empty = ~fin
    assert np.all(og[both_empty] == 0)
    # one rounding to the storage dtype of an fp32 combination
    eps = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    assert np.all(np.abs(og - ro) <= eps * np.abs(ro) + 1e-6 + 4 * eps * np.abs(ro).max() * 1e-3)
    # a side with lse = -inf leaves the other exactly
    only_a = np.isneginf(f64(lb)) & np.isfinite(f64(la))
    assert np.array_equal(og[only_a], f64(oa)[only_a])


def test_accumulate_bits_select_the_outputs():
    """accumulate={"dq"}: dq is added into, dk / dv are written as by the plain call."""
    import bwd_thd_varlen_amd as A
    L = [100, 37]
    rng = np.random.default_rng(63)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16).cuda()
    T = sum(L)
    q, k, v, do = mk(T, 4, 64), mk(T, 2, 64), mk(T, 2, 64), mk(T, 4, 64)
    cu = cu_dev(np.concatenate([[0], np.cumsum(L)]))
    o, l = A.fwd(q, k, v, cu, cu, attn_mask_type="padding_causal")
    g = A.bwd(q, k, v, o, do, l, cu, cu, attn_mask_type="padding_causal")
    base = mk(T, 4, 64)
    dq = base.clone()
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    A.bwd_chunk(q, k, v, o, do, l, cu, cu, dq=dq, dk=dk, dv=dv, accumulate={"dq"})
    assert torch.equal(dk, g[1]) and torch.equal(dv, g[2])
    want = (base.float() + g[0].float()).to(torch.bfloat16)
    assert (dq.float() - want.float()).abs().max().item() <= \
        want.float().abs().max().item() * 2.0 ** -7
    dq2 = torch.full_like(q, float("nan"))
    dk2, dv2 = torch.zeros_like(k), torch.zeros_like(v)
    A.bwd_chunk(q, k, v, o, do, l, cu, cu, dq=dq2, dk=dk2, dv=dv2, accumulate={"dkdv"})
    assert torch.equal(dq2, g[0])
    assert torch.equal(dk2, g[1]) and torch.equal(dv2, g[2])   # 0 + x rounds to x
