"""GPU parity for one causal sequence of 65536 tokens (512 query and key
tiles per head), against the oracle on exact sub-problems.

With the causal mask, query row i depends only on keys 0..i, so its output,
LSE and dQ are those of the one-query problem (q_i; K, V[0..i]) with the
bottom-right alignment (the query sees every key).  Key j only receives
gradient from queries i >= j, so dK and dV of the last 128 keys are those of
the problem (Q, dO[L-128..L); K, V) with the bottom-right alignment.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, assert_lse_close, cu_dev, f64

pytestmark = pytest.mark.gpu

L, HQ, HKV, D, TAIL = 65536, 8, 1, 128, 128


def test_single_sequence_65536_causal():
    import bwd_thd_varlen_amd as A
    rng = np.random.default_rng(2024)
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
    q, k, v, do = mk(L, HQ, D), mk(L, HKV, D), mk(L, HKV, D), mk(L, HQ, D)
    scale = 1.0 / math.sqrt(D)
    cu = cu_dev([0, L])
    print(f"[long] fwd+bwd of one {L}-token sequence", flush=True)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    kw = dict(attn_mask_type="padding_causal", softmax_scale=scale)
    o, l = A.fwd(qd, kd, vd, cu, cu, **kw)
    dq, dk, dv = A.bwd(qd, kd, vd, o, dod, l, cu, cu, **kw)
    torch.cuda.synchronize()

    for i in (0, 1, 127, 128, 4095, L // 2 + 77, L - 1):
        qi, doi = f64(q[i:i + 1]), f64(do[i:i + 1])
        kk, vv = f64(k[:i + 1]), f64(v[:i + 1])
        ro, rl = oracle.attn_fwd_seq(qi, kk, vv, scale, "bottom_right")
        rdq, _, _ = oracle.attn_bwd_seq(qi, kk, vv, doi, scale, "bottom_right")
        assert_close(f"out[{i}]", o[i:i + 1], ro, "bf16")
        assert_lse_close(l[i:i + 1], rl, np.ones(1, bool))
        if i == 0:
            # one visible key: P = 1 and dS = dP - Delta = 0, so dQ is exactly zero;
            # the kernels form Delta from the bf16-stored O, which leaves a residual
            # of the order of O's rounding
            assert float(dq[0].float().abs().max()) <= 1e-2
        else:
            assert_close(f"dq[{i}]", dq[i:i + 1], rdq, "bf16")

    qt, dot = f64(q[L - TAIL:]), f64(do[L - TAIL:])
    _, rdk, rdv = oracle.attn_bwd_seq(qt, f64(k), f64(v), dot, scale, "bottom_right")
    assert_close("dk[tail]", dk[L - TAIL:], rdk[L - TAIL:], "bf16")
    assert_close("dv[tail]", dv[L - TAIL:], rdv[L - TAIL:], "bf16")
