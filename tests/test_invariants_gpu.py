"""Bit-exact structural invariants on the GPU: exact zeros, determinism,
call-order independence under poisoned memory and allocator churn, no leak
from padding rows, and safe handling of bad cu_seqlens data."""
import numpy as np
import pytest
import torch

import workloads
from helpers import cu_dev, gpu_run, real_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import bwd_thd_varlen_amd as A
    A.lib()
    return A


def bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).clone()


def same_bits(a, b):
    return all(torch.equal(bits(x), bits(y)) for x, y in zip(a, b))


def poisoned_like(t):
    return torch.full_like(t, float("nan"))


def poisoned_workspace(case):
    import bwd_thd_varlen_amd as A
    n = A.workspace_size(case.batch, case.q.shape[0], case.k.shape[0], case.hq, case.hkv, case.d)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)     # every float in it reads as NaN, every int as -1
    return ws


def poisoned_run(case):
    q = case.q
    return gpu_run(case, workspace=poisoned_workspace(case),
                   out=poisoned_like(q.cuda()), lse=torch.full((q.shape[0], case.hq), float("nan"),
                                                                  device="cuda"),
                   dq=poisoned_like(q.cuda()), dk=poisoned_like(case.k.cuda()),
                   dv=poisoned_like(case.v.cuda()))


def test_repeat_calls_bitwise_identical(A):
    from test_parity_gpu import _ragged_case
    L, P = [300, 1, 129, 0, 257], [304, 8, 136, 8, 264]
    # the split kernels with odd counts of 32-column blocks (d 144, 208), unspread
    split = [_ragged_case(L, L, P, P, hq=4, hkv=2, d=d, causal=c, dtype="bf16", seed=d)
             for d, c in ((144, True), (208, False))]
    for case in (workloads.real_vs_padded(576, causal=True), workloads.gqa_d256_batched(),
                 workloads.mha_causal_lengths([256, 256]), *split):
        r1 = gpu_run(case)
        r2 = gpu_run(case)
        r3 = poisoned_run(case)
        assert same_bits(r1, r2), case.name
        assert same_bits(r1, r3), case.name


def _churn():
    """TE-2448 comment: a 16 MB fp32 block freed and an 8 MB bf16 block
    allocated between two backward passes."""
    w = torch.randn(4096, 1024, device="cuda")
    w2 = w.to(torch.bfloat16)
    del w
    return w2


def test_call_order_independence_two_step_example(A):
    c1, c2 = workloads.tiny_gqa_two_calls()
    a1 = poisoned_run(c1)
    keep = _churn()
    a2 = poisoned_run(c2)
    b2 = poisoned_run(c2)
    keep2 = _churn()
    b1 = poisoned_run(c1)
    torch.cuda.empty_cache()
    c2r = gpu_run(c2)
    assert same_bits(a1, b1)
    assert same_bits(a2, b2)
    assert same_bits(a2, c2r)
    # second call: first 4 (padded) kv tokens belong to a sequence with no query
    for t in (a2[3], a2[4]):
        assert int(torch.count_nonzero(bits(t[:4]))) == 0
    del keep, keep2


def test_call_order_with_shared_workspace_and_outputs(A):
    """Reusing one workspace and one set of output buffers across the two calls,
    in both orders, gives the same bits as fresh buffers."""
    c1, c2 = workloads.tiny_gqa_two_calls()
    ws = poisoned_workspace(c1)
    outs = dict(out=poisoned_like(c1.q.cuda()), lse=torch.full((12, 2), float("nan"), device="cuda"),
                dq=poisoned_like(c1.q.cuda()), dk=poisoned_like(c1.k.cuda()),
                dv=poisoned_like(c1.v.cuda()))
    fresh1, fresh2 = gpu_run(c1), gpu_run(c2)
    x = [t.clone() for t in gpu_run(c2, workspace=ws, **outs)]
    y = [t.clone() for t in gpu_run(c1, workspace=ws, **outs)]
    z = [t.clone() for t in gpu_run(c2, workspace=ws, **outs)]
    assert same_bits(x, fresh2) and same_bits(z, fresh2) and same_bits(y, fresh1)


def test_padding_rows_do_not_leak(A):
    """Redrawing every padding row (with noise, NaN and inf) changes no real row."""
    case = workloads.real_vs_padded(576, causal=False)
    r1 = gpu_run(case)
    T = case.q.shape[0]
    pad = ~real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, T)
    g = torch.Generator().manual_seed(123)
    for name in ("q", "k", "v", "dout"):
        t = getattr(case, name).clone()
        noise = torch.randn(t[pad].shape, generator=g).to(t.dtype) * 1000
        noise.view(-1)[::7] = float("nan")
        noise.view(-1)[::11] = float("inf")
        t[pad] = noise
        setattr(case, name, t)
    r2 = gpu_run(case)
    assert same_bits(r1, r2)


def test_zero_rows_exact(A):
    case = workloads.real_vs_padded(576, causal=True)
    o, l, dq, dk, dv = gpu_run(case)
    T = case.q.shape[0]
    pad = torch.as_tensor(~real_rows(case.cu_seqlens_q, case.cu_seqlens_q_padded, T), device="cuda")
    for t in (o, dq, dk, dv):
        assert int(torch.count_nonzero(bits(t[pad]))) == 0
    assert bool(torch.all(torch.isneginf(l[pad])))
    assert pad[-32:].all()    # the 32 trailing rows belong to no sequence


def test_empty_sequences_and_empty_batch(A):
    d, hq, hkv = 64, 4, 2
    T = 40
    q = torch.randn(T, hq, d, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(T, hkv, d, device="cuda", dtype=torch.bfloat16)
    v = torch.randn_like(k)
    do = torch.randn_like(q)
    # all sequences empty
    for cu in ([0, 0, 0], [0]):
        c = cu_dev(cu)
        cp = cu_dev([0, 20, 40][:len(cu)]) if len(cu) > 1 else cu_dev([0])
        out = poisoned_like(q)
        o, l = A.fwd(q, k, v, c, c, cp, cp, attn_mask_type="padding_causal", out=out)
        dq, dk, dv = A.bwd(q, k, v, o, do, l, c, c, cp, cp, attn_mask_type="padding_causal",
                           dq=poisoned_like(q), dk=poisoned_like(k), dv=poisoned_like(v))
        for t in (o, dq, dk, dv):
            assert int(torch.count_nonzero(bits(t))) == 0
        assert bool(torch.all(torch.isneginf(l)))


def test_bad_seqlens_data_sets_status_and_zero_outputs(A):
    d, hq, hkv, T = 32, 2, 1, 48
    q = torch.randn(T, hq, d, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(T, hkv, d, device="cuda", dtype=torch.bfloat16)
    v = torch.randn_like(k)
    do = torch.randn_like(q)
    bad_sets = [
        ([0, 30, 20], None),              # decreasing real boundaries
        ([0, 10, 20], [0, 8, 40]),        # real length above its padded slot
        ([0, 10, 20], [0, 16, 64]),       # slot beyond total rows
        ([0, 10, 20], [0, 32, 16]),       # decreasing padded boundaries
    ]
    for cu, cup in bad_sets:
        c = cu_dev(cu)
        cp = None if cup is None else cu_dev(cup)
        ws = torch.empty(A.workspace_size(2, T, T, hq, hkv, d), dtype=torch.uint8, device="cuda")
        o, l = A.fwd(q, k, v, c, c, cp, cp, out=poisoned_like(q), workspace=ws)
        assert A.read_device_status(ws) & A.DEV_BAD_SEQLENS
        dq, dk, dv = A.bwd(q, k, v, o, do, l, c, c, cp, cp, workspace=ws, dq=poisoned_like(q),
                           dk=poisoned_like(k), dv=poisoned_like(v))
        assert A.read_device_status(ws) & A.DEV_BAD_SEQLENS
        for t in (o, dq, dk, dv):
            assert int(torch.count_nonzero(bits(t))) == 0
    # and a good call on the same workspace clears the status
    c = cu_dev([0, 10, 20])
    ws = torch.empty(A.workspace_size(2, T, T, hq, hkv, d), dtype=torch.uint8, device="cuda")
    A.fwd(q, k, v, c, c, workspace=ws)
    assert A.read_device_status(ws) == 0


def test_binding_rejects_cpu_tensors(A):
    q = torch.randn(4, 1, 8, dtype=torch.bfloat16)
    with pytest.raises(A.AttnError):
        A.fwd(q, q, q, torch.tensor([0, 4], dtype=torch.int32), torch.tensor([0, 4], dtype=torch.int32))
