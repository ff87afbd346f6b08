"""Batches larger than the scheduler's 1024 threads: 3000 sequences, most of
them 0-96 tokens (empty query or key sides included) and 24 of 100-1000
tokens scattered among them, in padded slots, so that every loop over the
sequences takes several passes and the heaviest-first lists hold many
distinct work keys.  Compared in full with the oracle (every output on real
rows at the acceptance bar, every uncovered row +0.0 / -inf)."""
import numpy as np
import pytest
import torch

import workloads
from helpers import check_case

pytestmark = pytest.mark.gpu


def _case(mask, seed):
    rng = np.random.default_rng(seed)
    B, n_long = 3000, 24
    lq = rng.integers(0, 97, size=B)
    long_at = rng.choice(B, size=n_long, replace=False)
    lq[long_at] = rng.integers(100, 1001, size=n_long)
    if mask == "padding_causal":
        lk = lq.copy()
    else:
        lk = np.maximum(0, lq + rng.integers(-40, 41, size=B))
    lq[rng.choice(B, size=60, replace=False)] = 0    # sequences with no query
    lk[rng.choice(B, size=60, replace=False)] = 0    # and with no key
    pq = lq + rng.integers(0, 16, size=B)
    pk = lk + rng.integers(0, 16, size=B)
    hq, hkv, d = 4, 2, 64
    tq, tk = int(pq.sum()) + 7, int(pk.sum()) + 7      # a few rows past every slot
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(torch.bfloat16)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    causal = True if mask == "padding_causal" else "bottom_right"
    return workloads.Case(name=f"many_sequences_{mask}", q=mk(tq, hq, d), k=mk(tk, hkv, d),
                          v=mk(tk, hkv, d), dout=mk(tq, hq, d), cu_seqlens_q=cu(lq),
                          cu_seqlens_kv=cu(lk), cu_seqlens_q_padded=cu(pq),
                          cu_seqlens_kv_padded=cu(pk), scale=d ** -0.5, causal=causal,
                          dtype="bf16", max_seqlen_q=int(pq.max()), max_seqlen_kv=int(pk.max()))


@pytest.mark.parametrize("mask,seed", [("padding_causal", 3100), ("padding_causal_bottom_right", 3101)])
def test_three_thousand_sequences(mask, seed):
    case = _case(mask, seed)
    print(f"[many] {case.name}: B={case.batch} Tq={case.q.shape[0]} Tk={case.k.shape[0]}", flush=True)
    check_case(case)
