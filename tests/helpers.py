"""Shared test glue: run a workload through the GPU library and through the
CPU oracle, and compare them to the acceptance bar.

Acceptance for floating-point outputs on real rows: cosine >= 0.9999 and
max|gpu - ref| <= 2e-2 * max|ref| (bf16) or 5e-3 * max|ref| (fp16).  LSE is
fp32 end to end: |gpu - ref| <= 1e-3 + 1e-4 |ref|.  Rows outside the real
ranges must be exactly +0.0 (lse exactly -inf).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

TOL = {workloads.BF16: 2e-2, workloads.FP16: 5e-3}
COS_MIN = 0.9999


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def cu_dev(a, dev="cuda"):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=dev)


def real_rows(cu, cu_pad, total, other_cu=None):
    """Boolean mask of rows inside a real range (optionally only sequences whose
    other side is non-empty)."""
    m = np.zeros(total, dtype=bool)
    lens = np.diff(np.asarray(cu, np.int64))
    other = None if other_cu is None else np.diff(np.asarray(other_cu, np.int64))
    for b, (o, L) in enumerate(zip(np.asarray(cu_pad)[:-1], lens)):
        if other is not None and other[b] == 0:
            continue
        m[o:o + L] = True
    return m


def gpu_run(case, workspace=None, out=None, lse=None, dq=None, dk=None, dv=None,
            out_override=None, lse_override=None):
    """fwd then bwd through the library; returns CUDA tensors (out, lse, dq, dk, dv)."""
    import bwd_thd_varlen_amd as A
    q, k, v, do = (t.cuda() for t in (case.q, case.k, case.v, case.dout))
    cq, ck = cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv)
    cqp, ckp = cu_dev(case.cu_seqlens_q_padded), cu_dev(case.cu_seqlens_kv_padded)
    kw = dict(cu_seqlens_q_padded=cqp, cu_seqlens_kv_padded=ckp, max_seqlen_q=case.max_seqlen_q,
              max_seqlen_kv=case.max_seqlen_kv, attn_mask_type=case.mask_type,
              softmax_scale=case.scale, workspace=workspace)
    o, l = A.fwd(q, k, v, cq, ck, out=out, lse=lse, **kw)
    ob = o if out_override is None else out_override.cuda()
    lb = l if lse_override is None else lse_override.cuda()
    g = A.bwd(q, k, v, ob, do, lb, cq, ck, dq=dq, dk=dk, dv=dv, **kw)
    return (o, l) + tuple(g)


def oracle_run(case, mode="definition", out=None, lse=None):
    args = (case.cu_seqlens_q, case.cu_seqlens_kv, case.cu_seqlens_q_padded,
            case.cu_seqlens_kv_padded)
    o, l = oracle.attn_fwd(f64(case.q), f64(case.k), f64(case.v), *args, scale=case.scale,
                           causal=case.causal)
    g = oracle.attn_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.dout), *args,
                        scale=case.scale, causal=case.causal,
                        out=o if out is None else out, lse=l if lse is None else lse, mode=mode)
    return (o, l) + tuple(g)


def cosine(a, b):
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    if na == 0 or nb == 0:
        return 0.0
    return float(np.dot(a.ravel(), b.ravel()) / (na * nb))


def assert_close(name, gpu, ref, dtype, rows=None):
    g, r = f64(gpu), np.asarray(ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    if r.size == 0:
        return
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    mx = float(np.abs(r).max())
    err = float(np.abs(g - r).max())
    cos = cosine(g, r)
    assert cos >= COS_MIN, f"{name}: cosine {cos:.7f} < {COS_MIN}"
    assert err <= TOL[dtype] * max(mx, 1e-30), f"{name}: max err {err:.3e} > {TOL[dtype]}*{mx:.3e}"


def assert_lse_close(gpu, ref, rows):
    g, r = f64(gpu)[rows], np.asarray(ref)[rows]
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), "lse: -inf pattern differs"
    if fin.any():
        err = np.abs(g[fin] - r[fin])
        assert np.all(err <= 1e-3 + 1e-4 * np.abs(r[fin])), f"lse max err {err.max():.3e}"


def assert_exact_zero_rows(name, t, rows):
    """Rows selected by `rows` must be bit-exact +0.0."""
    if not rows.any():
        return
    sel = t[torch.as_tensor(rows, device=t.device)]
    bits = sel.contiguous().view(torch.int16 if sel.element_size() == 2 else torch.int32)
    assert int(torch.count_nonzero(bits)) == 0, f"{name}: uncovered rows are not +0.0"


def check_case(case, res=None, ref=None):
    """Full parity check of one workload (all rows)."""
    res = gpu_run(case) if res is None else res
    ref = oracle_run(case) if ref is None else ref
    o, l, dq, dk, dv = res
    ro, rl, rdq, rdk, rdv = ref
    Tq, Tk = case.q.shape[0], case.k.shape[0]
    qrows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, Tq, case.cu_seqlens_kv)
    krows = real_rows(case.cu_seqlens_kv, case.cu_seqlens_kv_padded, Tk, case.cu_seqlens_q)
    assert_close("out", o, ro, case.dtype, qrows)
    assert_lse_close(l, rl, qrows)
    assert_close("dq", dq, rdq, case.dtype, qrows)
    assert_close("dk", dk, rdk, case.dtype, krows)
    assert_close("dv", dv, rdv, case.dtype, krows)
    for name, t, rows in (("out", o, ~qrows), ("dq", dq, ~qrows), ("dk", dk, ~krows),
                          ("dv", dv, ~krows)):
        assert_exact_zero_rows(name, t, rows)
    lneg = f64(l)[~qrows]
    assert np.all(np.isneginf(lneg)), "lse of uncovered rows must be -inf"
    return res, ref
