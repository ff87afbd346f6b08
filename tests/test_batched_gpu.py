"""GPU parity of the batched layouts (bshd [b, s, h, d] and sbhd [s, b, h, d]
read in place by attn_fwd_batched / attn_bwd_batched).

Each case is also expressed in THD form (rows b*s + i, cu_seqlens_padded =
slot boundaries): the oracle runs on that form, and the batched results,
mapped to it, must pass the same acceptance bar as THD calls.  Because the
kernels' arithmetic for a (sequence, head) does not depend on where its rows
sit in memory, the batched results must also equal the THD call on the same
data bitwise.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from helpers import check_case, gpu_run

pytestmark = pytest.mark.gpu


def _to_thd(x, layout):
    """[b,s,...] or [s,b,...] -> [b*s, ...] (a copy for sbhd)."""
    if layout == "sbhd":
        x = x.transpose(0, 1)
    return x.reshape((x.shape[0] * x.shape[1],) + tuple(x.shape[2:])).contiguous()


def _from_thd(x, layout, b, s):
    x = x.reshape((b, s) + tuple(x.shape[1:]))
    return x.transpose(0, 1).contiguous() if layout == "sbhd" else x.contiguous()


def _batched_case(layout, b, sq, skv, lq, lk, hq, hkv, d, causal, seed, dtype="bf16"):
    """Batched tensors plus the equivalent THD workload case."""
    rng = np.random.default_rng(seed)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(td)
    q, do = mk(b * sq, hq, d), mk(b * sq, hq, d)
    k, v = mk(b * skv, hkv, d), mk(b * skv, hkv, d)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    lq = [sq] * b if lq is None else lq
    lk = [skv] * b if lk is None else lk
    case = workloads.Case(name=f"batched_{layout}", q=q, k=k, v=v, dout=do, cu_seqlens_q=cu(lq),
                          cu_seqlens_kv=cu(lk), cu_seqlens_q_padded=cu([sq] * b),
                          cu_seqlens_kv_padded=cu([skv] * b), scale=1 / math.sqrt(d),
                          causal=causal, dtype=dtype, max_seqlen_q=sq, max_seqlen_kv=skv)
    bt = {n: _from_thd(t, layout, b, s) for n, t, s in
          (("q", q, sq), ("k", k, skv), ("v", v, skv), ("dout", do, sq))}
    return case, bt


def _run_batched(case, bt, layout, b, sq, skv, full):
    import bwd_thd_varlen_amd as A
    q, k, v, do = (bt[n].cuda() for n in ("q", "k", "v", "dout"))
    kw = dict(layout=layout, attn_mask_type=case.mask_type, softmax_scale=case.scale)
    if not full:
        kw["cu_seqlens_q"] = torch.as_tensor(case.cu_seqlens_q, device="cuda")
        kw["cu_seqlens_kv"] = torch.as_tensor(case.cu_seqlens_kv, device="cuda")
    o, l = A.fwd_batched(q, k, v, **kw)
    dq, dk, dv = A.bwd_batched(q, k, v, o, do, l, **kw)
    assert l.shape == ((b, sq, case.hq) if layout == "bshd" else (sq, b, case.hq))
    return (_to_thd(o, layout), _to_thd(l, layout), _to_thd(dq, layout), _to_thd(dk, layout),
            _to_thd(dv, layout))


def _check(layout, b, sq, skv, lq, lk, hq, hkv, d, causal, seed, dtype="bf16"):
    case, bt = _batched_case(layout, b, sq, skv, lq, lk, hq, hkv, d, causal, seed, dtype)
    res = _run_batched(case, bt, layout, b, sq, skv, full=lq is None and lk is None)
    check_case(case, res=res)
    thd = gpu_run(case)
    for name, x, y in zip(("out", "lse", "dq", "dk", "dv"), res, thd):
        assert torch.equal(x, y), f"{name}: batched {layout} differs from the THD call"


@pytest.mark.parametrize("layout", ["bshd", "sbhd"])
@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
def test_batched_ragged_real_lengths(layout, causal):
    # slots of 200 queries / 260 keys; real lengths ragged, one empty sequence
    _check(layout, b=4, sq=200, skv=260, lq=[200, 131, 0, 77], lk=[260, 97, 50, 200], hq=8,
           hkv=2, d=128, causal=causal, seed=40)


@pytest.mark.parametrize("layout", ["bshd", "sbhd"])
@pytest.mark.parametrize("d", [32, 64, 256])
def test_batched_full_slots_head_dims(layout, d):
    _check(layout, b=3, sq=150, skv=150, lq=None, lk=None, hq=4, hkv=1, d=d, causal=True,
           seed=41 + d)


def test_sbhd_fp16_bottom_right():
    _check("sbhd", b=5, sq=70, skv=140, lq=[70, 33, 70, 1, 64], lk=[140, 140, 20, 5, 64], hq=6,
           hkv=3, d=64, causal="bottom_right", seed=42, dtype="fp16")


@pytest.mark.parametrize("outliers", [False, True])
def test_te3216_shape_as_native_sbhd(outliers):
    """The sbhd [384, 2, 16, 256] causal GQA workload run in its own layout:
    equal (bitwise) to its THD form and within the bar of the oracle."""
    case = workloads.gqa_d256_batched(outliers=outliers)
    S, B = 384, 2
    bt = {n: _from_thd(getattr(case, n), "sbhd", B, S) for n in ("q", "k", "v", "dout")}
    res = _run_batched(case, bt, "sbhd", B, S, S, full=True)
    check_case(case, res=res)
    thd = gpu_run(case)
    for name, x, y in zip(("out", "lse", "dq", "dk", "dv"), res, thd):
        assert torch.equal(x, y), name
