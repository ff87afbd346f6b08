"""A seeded sweep over random problem shapes, each compared in full with the
oracle (every output at the acceptance bar on real rows, every uncovered row
exactly +0.0 and -inf): ragged lengths with empty query or key sides, real !=
padded slots, rows past every slot, Lq != Lk, GQA ratios 1..8, head dims
8..256, bf16 and fp16, all three masks and a range of softmax scales.  The
configurations are drawn once from a fixed seed, so a failure names a
reproducible case."""
import numpy as np
import pytest
import torch

import workloads
from helpers import check_case

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    batch = int(rng.integers(1, 7))
    lq = rng.integers(0, 300, size=batch)
    lk = rng.integers(0, 300, size=batch)
    mask = ["padding", "padding_causal", "padding_causal_bottom_right"][i % 3]
    if mask == "padding_causal" and i % 2 == 0:
        lk = lq.copy()                       # the pages' causal case: Lq == Lk
    if i % 5 == 0:
        lq[rng.integers(0, batch)] = 0       # a sequence with no query
    if i % 7 == 0:
        lk[rng.integers(0, batch)] = 0       # a sequence with no key
    pq = lq + rng.integers(0, 40, size=batch)
    pk = lk + rng.integers(0, 40, size=batch)
    extra = int(rng.integers(0, 50)) if i % 4 == 0 else 0   # rows past every slot
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 8]))
    d = int(8 * rng.integers(1, 33))
    dtype = "fp16" if i % 3 == 1 else "bf16"
    scale = float(rng.uniform(0.05, 0.3)) if i % 2 else d ** -0.5
    return dict(lq=lq, lk=lk, pq=pq, pk=pk, extra=extra, hq=hkv * group, hkv=hkv, d=d,
                dtype=dtype, scale=scale, mask=mask, seed=2000 + i)


def _case(c):
    rng = np.random.default_rng(c["seed"])
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[c["dtype"]]
    tq, tk = int(c["pq"].sum()) + c["extra"], int(c["pk"].sum()) + c["extra"]
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s, dtype=np.float32)).to(td)
    cu = lambda a: np.concatenate([[0], np.cumsum(a)]).astype(np.int32)
    causal = {"padding": False, "padding_causal": True,
              "padding_causal_bottom_right": "bottom_right"}[c["mask"]]
    return workloads.Case(name="sweep", q=mk(tq, c["hq"], c["d"]), k=mk(tk, c["hkv"], c["d"]),
                          v=mk(tk, c["hkv"], c["d"]), dout=mk(tq, c["hq"], c["d"]),
                          cu_seqlens_q=cu(c["lq"]), cu_seqlens_kv=cu(c["lk"]),
                          cu_seqlens_q_padded=cu(c["pq"]), cu_seqlens_kv_padded=cu(c["pk"]),
                          scale=c["scale"], causal=causal, dtype=c["dtype"],
                          max_seqlen_q=int(c["pq"].max()), max_seqlen_kv=int(c["pk"].max()))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = _draw(i)
    print(f"[sweep] case {i}: B={len(c['lq'])} lq={c['lq'].tolist()} lk={c['lk'].tolist()} "
          f"hq={c['hq']} hkv={c['hkv']} d={c['d']} {c['dtype']} {c['mask']} "
          f"scale={c['scale']:.3f} extra={c['extra']}", flush=True)
    check_case(_case(c))
