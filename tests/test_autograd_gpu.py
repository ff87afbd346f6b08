"""The autograd op runs the same entry points: its outputs and gradients equal
the direct fwd / bwd calls bitwise, and a causal GQA case with padding matches
the oracle."""
import math

import numpy as np
import pytest
import torch

from helpers import assert_close, cu_dev, f64, oracle_run, real_rows
import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mask,p", [("padding_causal", 0.0), ("padding", 0.0),
                                    ("padding_causal", 0.2)])
def test_autograd_equals_direct_calls(mask, p):
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(80)
    L, P = [70, 129, 5], [72, 130, 8]
    T = sum(P)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16).cuda()
    q, k, v, do = mk(T, 8, 64), mk(T, 2, 64), mk(T, 2, 64), mk(T, 8, 64)
    cu = cu_dev(np.concatenate([[0], np.cumsum(L)]))
    cp = cu_dev(np.concatenate([[0], np.cumsum(P)]))
    kw = dict(cu_seqlens_q_padded=cp, cu_seqlens_kv_padded=cp, attn_mask_type=mask,
              dropout_p=p, rng_seed=7, rng_offset=1)
    qa, ka, va = (t.clone().requires_grad_() for t in (q, k, v))
    out = A.attention_thd(qa, ka, va, cu, cu, **kw)
    out.backward(do)
    o, l = A.fwd(q, k, v, cu, cu, **kw)
    dq, dk, dv = A.bwd(q, k, v, o, do, l, cu, cu, **kw)
    assert torch.equal(out.detach(), o)
    for a, b in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        assert torch.equal(a, b)


def test_autograd_against_oracle():
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(81)
    L, P = [100, 37], [112, 40]
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
    T = sum(P)
    case = workloads.Case(name="autograd", q=mk(T, 4, 128), k=mk(T, 2, 128), v=mk(T, 2, 128),
                          dout=mk(T, 4, 128), cu_seqlens_q=cu(L), cu_seqlens_kv=cu(L),
                          cu_seqlens_q_padded=cu(P), cu_seqlens_kv_padded=cu(P),
                          scale=1 / math.sqrt(128), causal=True, dtype="bf16")
    q, k, v = (t.cuda().requires_grad_() for t in (case.q, case.k, case.v))
    out = A.attention_thd(q, k, v, cu_dev(case.cu_seqlens_q), cu_dev(case.cu_seqlens_kv),
                          cu_dev(case.cu_seqlens_q_padded), cu_dev(case.cu_seqlens_kv_padded))
    (out.float() * case.dout.cuda().float()).sum().backward()
    ro, _, rdq, rdk, rdv = oracle_run(case)
    rows = real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, T)
    assert_close("out", out.detach(), ro, "bf16", rows)
    assert_close("dq", q.grad, rdq, "bf16", rows)
    assert_close("dk", k.grad, rdk, "bf16", rows)
    assert_close("dv", v.grad, rdv, "bf16", rows)
